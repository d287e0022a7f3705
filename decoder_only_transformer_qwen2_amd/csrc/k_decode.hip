// Kernels of one decode step (one new token per sequence, B <= 32 sequences).
//
// What a step computes is the decoder block of "LLM Speedrun: Architecture"
// (sections "Normalization", "Attention", "Grouped Query Attention GQA",
// "Split-half RoPE implementation", "Introducing bias", "Decoding") for one
// row per sequence, reading past keys and values from the preallocated cache
// ("augur").  How it is laid out is specific to this GPU:
//
//  * Kernel boundaries are the only cheap device-wide synchronisation here,
//    and a device-scope fence per workgroup is expensive, so no workgroup
//    waits on another (the norm hand-off counts arrivals, without a fence).  Projections split K over workgroups and add their
//    partial sums with 64-bit integer atomics on a fixed-point copy of the
//    value (32 fractional bits).  Integer addition is associative, so the
//    result does not depend on arrival order (deterministic), and no fence is
//    needed: the consumer is the next kernel.
//  * Each consumer finishes the step its input belongs to while staging its
//    operand: attention applies bias and RoPE to the q/k/v sums (and writes
//    k and v into the cache), the o projection merges split-KV partials (one
//    or two rows), and for one or two rows every projection computes the
//    RMSNorm of its own operand.
//  * One or two rows: per layer three kernels, the q/k/v projection, attention
//    merged with the o projection (short contexts; split-KV attention + o
//    projection past them) and the whole MLP (dec_mlp32_kernel).  The
//    residual is two fixed-point replicas (value = their sum) so that the
//    MLP's workgroups, which all add into every value of a row, spread their
//    atomics; it ping-pongs between two buffers around the MLP.
//  * More than two rows: the projections (gate/up without a K split, SwiGLU
//    in its epilogue), split-KV attention on the matrix cores
//    (dec_attn_mfma_kernel) and a merge kernel; the residual projections hand
//    the next RMSNorm its operand (norm_tail), so no norm kernel runs.
//  * Every load of a kernel's first phase is issued before any is consumed
//    (clamped addresses and selects rather than per-lane branches).
//  * Accumulators are cleared by an earlier kernel of the same step, so the
//    step needs no memset and replays as a graph.
#include "qw_internal.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

namespace qw {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float FIX_ONE = 4294967296.0f;            // 2^32
constexpr float FIX_INV = 2.3283064365386963e-10f;  // 2^-32
constexpr float LOG2E = 1.4426950408889634f;
constexpr int CH = 256;                             // k per staged chunk
constexpr int MERGE_MAX_S = 16;                     // split-KV partials merged per head

// A fixed-point value spans +-2^31.  Every addend is checked against 2^23
// (so no sum of the at most a few hundred addends of one value can wrap);
// one beyond it, or NaN, sets kFlagFixRange in the model's status word
// (qw_check_numerics) and is clamped so the conversion stays defined.
constexpr float FIX_ADDEND_MAX = 8388608.0f;        // 2^23
__device__ __forceinline__ long long to_fix(float v, int *flag) {
  if (!(fabsf(v) <= FIX_ADDEND_MAX)) atomicOr(flag, kFlagFixRange);
  v = fminf(fmaxf(v, -1.0e9f), 1.0e9f);
  return __float2ll_rn(v * FIX_ONE);
}
__device__ __forceinline__ float from_fix(long long q) { return (float)q * FIX_INV; }
__device__ __forceinline__ void fix_add(long long *p, float v, int *flag) {
  atomicAdd(reinterpret_cast<unsigned long long *>(p), (unsigned long long)to_fix(v, flag));
}
__device__ __forceinline__ f16x8 load8(const f16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

// Workgroup barrier that publishes LDS writes only: waits for this wave's LDS
// operations (lgkmcnt 0) but leaves its global loads in flight, where
// __syncthreads would first wait for every outstanding load (vmcnt 0).  The
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8 or 16; a group never
// crosses a 16-lane row), every lane ending with its group's sum.  DPP moves
// (VALU operands read from another lane of the row): swap neighbours, swap
// pairs, mirror each half-row, mirror the row.  A shuffle would go through the
// LDS crossbar (ds_bpermute) once per step.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
  auto mv = [](float x, int ctrl) -> float {
    switch (ctrl) {
      case 0xB1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
      case 0x4E: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
      case 0x141: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
    }
  };
  if constexpr (N >= 2) v += mv(v, 0xB1);    // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) v += mv(v, 0x4E);    // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) v += mv(v, 0x141);   // row_half_mirror
  if constexpr (N >= 16) v += mv(v, 0x140);  // row_mirror
  return v;
}
// Loads in these kernels are issued unconditionally from an address clamped
// into range, and a lane outside the range then selects zero (or its result
// is never stored).  A per-lane condition around the load itself becomes an
// exec-mask branch per load, which keeps the compiler from issuing a wave's
// loads back to back.

// Clear n int64 values, spread over `parts` cooperating workgroups.
__device__ __forceinline__ void clear_share(long long *p, int64_t n, int part, int parts) {
  if (!p) return;
  const int64_t per = (n + parts - 1) / parts;
  const int64_t lo = (int64_t)part * per, hi = min(n, lo + per);
  for (int64_t e = lo + threadIdx.x; e < hi; e += blockDim.x) p[e] = 0;
}

// ---------------------------------------------------------------- last arrival
// A result that needs every workgroup of a kernel: the workgroup that arrives
// last at a counter finishes it.  Everything it reads from the others was
// written with device-scope atomics (performed where every XCD sees them) and
// is read with device-scope atomic loads (which bypass non-coherent caches);
// each wave waits for its own atomics to be acknowledged before the count, so
// the count orders them.  A device-scope release fence would do the same but
// also writes back the whole L2 of the XCD: about 15 us more per projection
// launch at 32 rows, measured.
__device__ __forceinline__ long long ld_coherent(const long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// After this workgroup's device-scope writes: true in the workgroup that
// brings counter *c to n (which resets it for the next launch).  Uniform.
__device__ __forceinline__ bool arrive_last(int *c, int n) {
  __shared__ int s_last;
  wait_vmcnt<0>();                  // this wave's writes are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const int last = atomicAdd(c, 1) == n - 1;
    if (last) atomicExch(c, 0);
    s_last = last;
  }
  __syncthreads();
  return s_last;
}

// ---------------------------------------------------------------- RMSNorm hand-off
// Batched steps (more than two rows) have no kernel of their own for the
// RMSNorm ("LLM Speedrun: Architecture", "Normalization").  1/rms of a row
// needs the whole finished row, which only exists once every workgroup of the
// producing projection has added its share (fixed-point atomics).  So the
// workgroup that finishes a block of columns last writes the block's
// u = f16(x * w) and the sum of x^2 of each row over the block; the next
// projection multiplies u by its weights and scales output row b by
// 1/sqrt(sum_blocks / H + eps), which is the same product reassociated.  The
// sums are added in a fixed order, so the result does not depend on which
// workgroup came last.

// Consumer side: the partial sums are loaded at the start (consumed at the
// end, so their latency hides behind the weights) and reduced to 1/rms per
// row in LDS.  Thread t takes a run of C = round_up(ceil(parts / TPR), 4)
// parts of row t % 32, from part C (t / 32), as float4 loads (a row holds
// kNormPartsMax, so every load stays in it; parts past `parts` count zero).
template <int NT>
struct RowRstd {
  static constexpr int TPR = NT / 32;
  static constexpr int PER4 = (kNormPartsMax / TPR + 3) / 4;
  float4 v[PER4];
  int base = 0;
  __device__ __forceinline__ void load(const RowNormIn &n, int M) {
    const int b = threadIdx.x % 32, sub = threadIdx.x / 32;
    const int run = ((n.parts + TPR - 1) / TPR + 3) & ~3;     // uniform
    base = min(sub * run, kNormPartsMax - 4 * PER4);
    const float4 *p = reinterpret_cast<const float4 *>(n.ss + (int64_t)min(b, M - 1) * n.ss_ld + base);
#pragma unroll
    for (int t = 0; t < PER4; ++t) {
      v[t] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * t < run) v[t] = p[t];                            // uniform condition
    }
  }
  // every thread calls it; s_rstd[b] holds 1/rms of row b afterwards
  __device__ __forceinline__ void finish(const RowNormIn &n, float (*s_part)[32], float *s_rstd) {
    const int b = threadIdx.x % 32, sub = threadIdx.x / 32;
    const int run = ((n.parts + TPR - 1) / TPR + 3) & ~3;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < PER4; ++k) {
      const float e[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int part = base + 4 * k + q;
        if (4 * k + q < run && part >= sub * run && part < n.parts) t += e[q];
      }
    }
    s_part[sub][b] = t;
    __syncthreads();
    if (threadIdx.x < 32) {
      float tot = 0.f;
#pragma unroll
      for (int k = 0; k < TPR; ++k) tot += s_part[k][threadIdx.x];
      s_rstd[threadIdx.x] = 1.0f / sqrtf(tot / n.dim + n.eps);
    }
    __syncthreads();
  }
};

// Producer side, after a FixAdd projection's residual additions: the last of
// the gridDim.y K slices of column block nblk (RB columns from n0) forms u and
// the block's sums of squares.  s_buf: RB * BT floats of free LDS.
template <int RB, int BT, int NT>
__device__ __forceinline__ void norm_tail(const DecGemvArgs &a, int n0, int nblk, float *s_buf) {
  // K split: the residual was updated by device-scope atomics of gridDim.y
  // workgroups; otherwise by this workgroup alone (plain stores, visible to
  // it after the barrier)
  const bool split = gridDim.y > 1;
  if (split) {
    if (!arrive_last(a.nout.counters + nblk, gridDim.y)) return;
  } else {
    __syncthreads();
  }
  for (int e = threadIdx.x; e < RB * BT; e += NT) {
    const int nl = e % RB, b = e / RB, n = n0 + nl;
    float sq = 0.f;
    if (n < a.N && b < a.M) {
      long long q = 0;
#pragma unroll
      for (int r = 0; r < kXReps; ++r) {
        const long long *p = a.out_fix + r * a.nout.rep_stride + (int64_t)b * a.ldo + n;
        q += split ? ld_coherent(p) : *p;
      }
      const float x = from_fix(q);
      ((f16 *)a.nout.u)[a.nout.tiled ? tile_off(b, n, a.N) : (int64_t)b * a.N + n] = (f16)(x * a.nout.w[n]);
      sq = x * x;
    }
    s_buf[b * RB + nl] = sq;
  }
  __syncthreads();
  if ((int)threadIdx.x < a.M) {
    float t = 0.f;
    for (int nl = 0; nl < RB; ++nl) t += s_buf[threadIdx.x * RB + nl];
    a.nout.ss[(int64_t)threadIdx.x * a.nout.ss_ld + nblk] = t;
  }
}

// ---------------------------------------------------------------- begin / norm / end
// x_fix[b] = embedding row of ids[b] (its exact value, in fixed point); clears
// the q/k/v and gate/up accumulators for the first layer.  With nout.w set
// (batched steps) also the first layer's u = f16(x * w) and sum of x^2.
__global__ void __launch_bounds__(256) dec_embed_kernel(const int32_t *ids, const f16 *emb, float emb_scale, int H,
                                                        int V, long long *x_fix, int *bad, long long *clr0,
                                                        int64_t n0, long long *clr1, int64_t n1, RowNormOut nout) {
  const int b = blockIdx.x;
  int id = ids[b];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) atomicOr(bad, kFlagBadId);
    id = 0;
  }
  const f16 *row = emb + (int64_t)id * H;
  float ss = 0.f;
  for (int c = threadIdx.x; c < H; c += blockDim.x) {
    const long long q = to_fix((float)row[c] * emb_scale, bad);
    x_fix[(int64_t)b * H + c] = q;
    if (nout.w) {
      const float x = from_fix(q);
      ((f16 *)nout.u)[nout.tiled ? tile_off(b, c, H) : (int64_t)b * H + c] = (f16)(x * nout.w[c]);
      ss += x * x;
    }
  }
  if (nout.w) {
    __shared__ float red[4];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) nout.ss[(int64_t)b * nout.ss_ld] = red[0] + red[1] + red[2] + red[3];
  }
  clear_share(clr0, n0, b, gridDim.x);
  clear_share(clr1, n1, b, gridDim.x);
}

// u[b] = f16(x[b] / sqrt(mean(x[b]^2) + eps) * w): before the LM head of one or
// two rows, and for larger batches whose residual projections cannot hand the
// norm on (more column blocks than kNormPartsMax).
__global__ void __launch_bounds__(256) dec_norm_kernel(const long long *x_fix, int64_t rep_stride, int H,
                                                       const float *w, float eps, f16 *u) {
  const int b = blockIdx.x;
  __shared__ float red[4];
  const long long *xr = x_fix + (int64_t)b * H;
  float ss = 0.f;
  for (int c0 = 0; c0 < H; c0 += 256 * 8) {
    long long v[8];
    long long vr[kXReps][8];
#pragma unroll
    for (int r = 0; r < kXReps; ++r)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int c = c0 + t * 256 + threadIdx.x;
        const long long q = xr[r * rep_stride + min(c, H - 1)];
        vr[r][t] = c < H ? q : 0;
      }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      v[t] = vr[0][t];
#pragma unroll
      for (int r = 1; r < kXReps; ++r) v[t] += vr[r][t];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float f = from_fix(v[t]);
      ss += f * f;
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  for (int c = threadIdx.x; c < H; c += 256) {
    long long q = xr[c];
#pragma unroll
    for (int r = 1; r < kXReps; ++r) q += xr[r * rep_stride + c];
    u[(int64_t)b * H + c] = (f16)(from_fix(q) * inv * w[c]);
  }
}

// Reduce the LM head's per-block (max, index) pairs: lowest index among equal
// maxima.  Advances the row's device-side position.
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
    pos_dev[b] += 1;
  }
}

// For more than two rows the o projection takes an f16 operand formed once,
// rather than in every row-block workgroup's prologue: o[b, h] = merge of the
// S split-KV partials of head h (one workgroup per (head, row), one thread
// per dimension).  (The gate/up projection writes silu(gate) * up itself.)
// Dimension d of one head's output from its S split-KV partials (max m, sum l,
// unnormalised output o), partials st0 .. st0 + S - 1.
__device__ __forceinline__ float merge_splits(const float *pm, const float *pl, const float *po, int64_t st0, int S,
                                              int hd, int d) {
  float m[MERGE_MAX_S], l[MERGE_MAX_S], v[MERGE_MAX_S];
#pragma unroll
  for (int sp = 0; sp < MERGE_MAX_S; ++sp) {
    const int64_t st = st0 + min(sp, S - 1);
    m[sp] = pm[st];
    l[sp] = pl[st];
    v[sp] = po[st * hd + d];
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < MERGE_MAX_S; ++sp)
    if (sp < S) M = fmaxf(M, m[sp]);
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int sp = 0; sp < MERGE_MAX_S; ++sp) {
    const float c = (sp < S && m[sp] != -INFINITY) ? exp2f(m[sp] - M) : 0.f;
    L = fmaf(c, l[sp], L);
    O = fmaf(c, v[sp], O);
  }
  return O / L;
}

__global__ void __launch_bounds__(128) dec_merge_kernel(const float *pm, const float *pl, const float *po, int S, int nq,
                                                        int hd, f16 *o, int tiled) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  if (d >= hd) return;
  const int qd = nq * hd;
  o[tiled ? tile_off(b, h * hd + d, qd) : (int64_t)b * qd + (int64_t)h * hd + d] =
      (f16)merge_splits(pm, pl, po, ((int64_t)b * nq + h) * S, S, hd, d);
}

// ---------------------------------------------------------------- projections
// out[b, n] (+)= sum_k act[b, k] * W[n, k] * scale for b < M <= 16 * NB.
// One wave = 16 weight rows x a K slice; a workgroup = 4 waves = 64 rows;
// gridDim.y = K slices.  The operand slice is produced once per workgroup
// into LDS, CH columns at a time, by one of the operand modes below; the
// weight rows of the next chunk are already in flight while a chunk is
// staged.  MFMA: weights are the A operand (16 rows), activations the B
// operand (16 batch rows); unit t of a chunk gives lane group g the 8
// columns 32t + 8g .. 32t + 8g + 7.
enum class DecAct : int { F16 = 0, NormFix = 1, SwiGLUFix = 2, AttnMerge = 3 };
enum class DecOut : int { FixAdd = 0, Logits = 1, SwiGLUOut = 2 };

// ROLE only separates launches in profiles (the gate/up projection gets its
// own symbol); it does not change the code.
template <int NB, DecAct AM, DecOut OM, int ROLE, int NFP = 1>
__global__ void __launch_bounds__(256) dec_gemv_kernel(DecGemvArgs a) {
  constexpr int BT = 16 * NB;
  __shared__ f16 s_act[BT][CH + 8];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int nblk = blockIdx.x, split = blockIdx.y;
  const int row = nblk * 64 + wave * 16 + i;
  const bool row_ok = row < a.N;
  const f16 *W = (const f16 *)a.W + (int64_t)(row_ok ? row : 0) * a.K;
  // unit-tiled weights: the wave's 16 rows are row block 4 nblk + wave
  const f16 *Wtl = (const f16 *)a.W + (int64_t)(nblk * 4 + wave) * (a.K >> 5) * 512 + 8 * lane;
  const int k0 = split * a.units_per_split * 32;
  const int k1 = min(a.K, k0 + a.units_per_split * 32);
  const f16x8 zero = {};

  // side job: clear an accumulator of the next layer, shared by all workgroups
  if (a.clear)
    clear_share(a.clear, a.clear_n, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  // LM head of a batched step: operand u without 1/rms (row sums of squares
  // loaded now, needed at the end)
  constexpr bool kRowScale = OM == DecOut::Logits && AM == DecAct::F16;
  const bool nrm = kRowScale && a.nin.ss != nullptr;
  RowRstd<256> rr;
  if (nrm) rr.load(a.nin, a.M);

  f16x8 w[8];
  auto load_w = [&](int kc) {
    // units past the chunk load a clamped address and are never multiplied
    // (a condition around the load would become a branch per load); rows >= N
    // are never stored
    const int nu = min(8, (k1 - kc) >> 5);
#pragma unroll
    for (int t = 0; t < 8; ++t)
      w[t] = a.w_tiled ? load8(Wtl + (int64_t)((kc >> 5) + min(t, nu - 1)) * 512)
                       : load8(W + kc + 32 * min(t, nu - 1) + 8 * g);
  };
  // with the norm in the prologue the residual rows are loaded first (the
  // norm then runs while the weights arrive)
  if constexpr (AM != DecAct::NormFix) load_w(k0);

  // NormFix: the whole normalised row (1 or 2 rows) is built once in LDS.
  // Every thread loads its share of the row and of the norm weight up front
  // (one memory round trip), then one block reduction gives 1/rms.
  constexpr int NF_ROWS = 2, NF_PER = NFP;    // rows, values per thread (K <= 256 NFP)
  __shared__ f16 s_row[(AM == DecAct::NormFix) ? NF_ROWS : 1][(AM == DecAct::NormFix) ? 256 * NF_PER : 8];
  if constexpr (AM == DecAct::NormFix) {
    __shared__ float s_red[4][NF_ROWS];
    float xv[NF_ROWS][NF_PER], wv[NF_PER];
#pragma unroll
    for (int t = 0; t < NF_PER; ++t) {
      const int c = t * 256 + tid;
      const float w = a.norm_w[min(c, a.K - 1)];
      wv[t] = c < a.K ? w : 0.f;
    }
    // all replicas of the rows in one batch of loads (clamped addresses)
    long long qr[kXReps][NF_ROWS][NF_PER];
#pragma unroll
    for (int r = 0; r < kXReps; ++r)
#pragma unroll
      for (int b = 0; b < NF_ROWS; ++b)
#pragma unroll
        for (int t = 0; t < NF_PER; ++t) {
          const int c = t * 256 + tid;
          const long long v = a.x_fix[r * a.x_rep_stride + (int64_t)min(b, a.M - 1) * a.lda + min(c, a.K - 1)];
          // masked arithmetically: a select on the (uniform) row test becomes
          // a branch per load, and the loads are then serialised
          qr[r][b][t] = v & -(long long)((b < a.M) & (c < a.K));
        }
    __builtin_amdgcn_sched_barrier(0);
    load_w(k0);
    __builtin_amdgcn_sched_barrier(0);
    long long q[NF_ROWS][NF_PER];
#pragma unroll
    for (int b = 0; b < NF_ROWS; ++b)
#pragma unroll
      for (int t = 0; t < NF_PER; ++t) {
        q[b][t] = qr[0][b][t];
#pragma unroll
        for (int r = 1; r < kXReps; ++r) q[b][t] += qr[r][b][t];
      }
#pragma unroll
    for (int b = 0; b < NF_ROWS; ++b)
#pragma unroll
      for (int t = 0; t < NF_PER; ++t) xv[b][t] = from_fix(q[b][t]);
#pragma unroll
    for (int b = 0; b < NF_ROWS; ++b) {
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < NF_PER; ++t) ss += xv[b][t] * xv[b][t];
      ss = wave_sum(ss);
      if (lane == 0) s_red[wave][b] = ss;
    }
    lds_barrier();                 // the weights stay in flight
#pragma unroll
    for (int b = 0; b < NF_ROWS; ++b) {
      const float inv = 1.0f / sqrtf((s_red[0][b] + s_red[1][b] + s_red[2][b] + s_red[3][b]) / (float)a.K + a.eps);
#pragma unroll
      for (int t = 0; t < NF_PER; ++t) {
        const int c = t * 256 + tid;
        if (c < a.K) s_row[b][c] = (f16)(xv[b][t] * inv * wv[t]);
      }
    }
    lds_barrier();
  }

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = k0; kc < k1; kc += CH) {
    const int ck = min(CH, k1 - kc);
    // the previous chunk's LDS reads are done (NormFix reads only s_row, which
    // stays as the prologue published it)
    if (AM != DecAct::NormFix && kc != k0) __syncthreads();
    // ---- stage act[b][kc .. kc + ck) for b < M
    if constexpr (AM == DecAct::AttnMerge) {
      // merge of the split-KV partials: each element loads its head's S
      // (max, sum) pairs and its S partial outputs together (one round trip)
      const int hd = a.head_dim, S = a.attn_splits;
#pragma unroll 2
      for (int e = tid; e < a.M * ck; e += 256) {
        const int b = e / ck, kk = e % ck, k = kc + kk;
        const int h = k / hd, d = k % hd;
        const int64_t st0 = ((int64_t)b * a.n_heads + h) * S;
        float pm[MERGE_MAX_S], pl[MERGE_MAX_S], po[MERGE_MAX_S];
#pragma unroll
        for (int sp = 0; sp < MERGE_MAX_S; ++sp) {
          if (sp < S) {
            pm[sp] = a.part_m[st0 + sp];
            pl[sp] = a.part_l[st0 + sp];
            po[sp] = a.part_o[(st0 + sp) * hd + d];
          }
        }
        float M = -INFINITY;
#pragma unroll
        for (int sp = 0; sp < MERGE_MAX_S; ++sp)
          if (sp < S) M = fmaxf(M, pm[sp]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int sp = 0; sp < MERGE_MAX_S; ++sp) {
          if (sp < S) {
            const float c = (pm[sp] == -INFINITY) ? 0.f : exp2f(pm[sp] - M);
            L = fmaf(c, pl[sp], L);
            O = fmaf(c, po[sp], O);
          }
        }
        s_act[b][kk] = (f16)(O / L);
      }
    } else if constexpr (AM == DecAct::F16) {
      for (int e = tid; e < a.M * (ck >> 3); e += 256) {
        const int b = e / (ck >> 3), kk = (e % (ck >> 3)) * 8;
        *reinterpret_cast<f16x8 *>(&s_act[b][kk]) = load8((const f16 *)a.act + (int64_t)b * a.lda + kc + kk);
      }
    } else if constexpr (AM == DecAct::NormFix) {
      // operand already in s_row
    } else {
      // features kc + kk; gate and up of feature f sit in GU_BLOCK-interleaved rows
      for (int e = tid; e < a.M * ck; e += 256) {
        const int b = e / ck, kk = e % ck, f = kc + kk;
        const long long *r2 = a.act_fix + (int64_t)b * a.lda + (f / GU_BLOCK) * 2 * GU_BLOCK + f % GU_BLOCK;
        const float gt = from_fix(r2[0]), up = from_fix(r2[GU_BLOCK]);
        s_act[b][kk] = (f16)(silu_f(gt) * up);
      }
    }
    if constexpr (AM != DecAct::NormFix) __syncthreads();
    // ---- multiply the chunk; fetch the next chunk's weights first
    f16x8 wc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) wc[t] = w[t];
    if (kc + CH < k1) load_w(kc + CH);
    const int nu = ck >> 5;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < nu) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int b = nb * 16 + i;
          const f16 *src = (AM == DecAct::NormFix) ? &s_row[b < NF_ROWS ? b : 0][kc + 32 * t + 8 * g]
                                                   : &s_act[b][32 * t + 8 * g];
          const f16x8 xl = *reinterpret_cast<const f16x8 *>(src);
          const f16x8 x = (b < a.M) ? xl : zero;
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wc[t], x, acc[nb], 0, 0, 0);
        }
      }
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
        if (nw + r < a.N) fix_add(a.out_fix + (int64_t)b * a.ldo + nw + r, acc[nb][r] * a.scale, a.num_flag);
    }
  } else if constexpr (OM == DecOut::SwiGLUOut) {
    // full K in this workgroup: waves 0/1 hold the gate/up rows of feature
    // block 2 nblk, waves 2/3 those of block 2 nblk + 1; they meet in LDS
    __shared__ float s_gu[4][16][BT];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_gu[wave][4 * g + r][nb * 16 + i] = acc[nb][r] * a.scale;
    __syncthreads();
    f16 *h = (f16 *)a.h_out;
    for (int e = tid; e < 2 * 16 * BT; e += 256) {
      const int pp = e / (16 * BT), rr = (e / BT) % 16, b = e % BT;
      const int f = nblk * 32 + pp * 16 + rr;
      if (b < a.M && f < a.N / 2) h[(int64_t)b * a.ldh + f] = (f16)(silu_f(s_gu[2 * pp][rr][b]) * s_gu[2 * pp + 1][rr][b]);
    }
  } else {
    // logits (optional copy) and this block's (max, lowest index) per batch row
    __shared__ float s_v[4][BT];
    __shared__ int s_i[4][BT];
    __shared__ float s_part[8][32], s_rstd[32];
    if (nrm) rr.finish(a.nin, s_part, s_rstd);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nb * 16 + i;
      const float rs = nrm ? s_rstd[b < 32 ? b : 0] : 1.f;
      float best = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = nw + r;
        const float v = nrm ? acc[nb][r] * a.scale * rs : acc[nb][r] * a.scale;
        if (n < a.N && b < a.M) {
          if (a.logits) a.logits[(int64_t)b * a.ldo + n] = v;
          if (v > best) { best = v; bi = n; }     // n increases with r
          if (!(fabsf(v) <= 3.4e38f)) atomicOr(a.num_flag, kFlagNonFinite);
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
      for (int w2 = 1; w2 < 4; ++w2)
        if (s_v[w2][tid] > best || (s_v[w2][tid] == best && s_i[w2][tid] < bi)) {
          best = s_v[w2][tid];
          bi = s_i[w2][tid];
        }
      a.arg_v[(int64_t)tid * gridDim.x + nblk] = best;
      a.arg_i[(int64_t)tid * gridDim.x + nblk] = bi;
    }
  }
}

// NormFix: one or two rows, the prologue sized to K (values per thread)
template <int ROLE, int NFP>
hipError_t launch_gemv_normfix(hipStream_t s, const DecGemvArgs &a, dim3 grid) {
  if (a.logits_mode)
    QW_LAUNCH((dec_gemv_kernel<1, DecAct::NormFix, DecOut::Logits, ROLE, NFP>), dim3(grid), dim3(256), 0, s, a);
  else
    QW_LAUNCH((dec_gemv_kernel<1, DecAct::NormFix, DecOut::FixAdd, ROLE, NFP>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int NB, int ROLE>
hipError_t launch_gemv_role(hipStream_t s, const DecGemvArgs &a, dim3 grid) {
  const DecAct am = (DecAct)a.act_mode;
  if (am == DecAct::NormFix) {
    if (a.M > 2 || a.K > 4096) return hipErrorInvalidValue;
    if (a.K <= 1024) return launch_gemv_normfix<ROLE, 4>(s, a, grid);
    if (a.K <= 2048) return launch_gemv_normfix<ROLE, 8>(s, a, grid);
    return launch_gemv_normfix<ROLE, 16>(s, a, grid);
  }
  if (a.logits_mode) {
    QW_LAUNCH((dec_gemv_kernel<NB, DecAct::F16, DecOut::Logits, ROLE>), dim3(grid), dim3(256), 0, s, a);
  } else if (a.swiglu_out) {
    if (am != DecAct::F16 || grid.y != 1) return hipErrorInvalidValue;
    QW_LAUNCH((dec_gemv_kernel<NB, DecAct::F16, DecOut::SwiGLUOut, ROLE>), dim3(grid), dim3(256), 0, s, a);
  } else {
    switch (am) {
      case DecAct::F16: QW_LAUNCH((dec_gemv_kernel<NB, DecAct::F16, DecOut::FixAdd, ROLE>), dim3(grid), dim3(256), 0, s, a); break;
      case DecAct::NormFix: break;
      case DecAct::SwiGLUFix: QW_LAUNCH((dec_gemv_kernel<NB, DecAct::SwiGLUFix, DecOut::FixAdd, ROLE>), dim3(grid), dim3(256), 0, s, a); break;
      case DecAct::AttnMerge: QW_LAUNCH((dec_gemv_kernel<NB, DecAct::AttnMerge, DecOut::FixAdd, ROLE>), dim3(grid), dim3(256), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

template <int NB>
hipError_t launch_gemv_nb(hipStream_t s, const DecGemvArgs &a, dim3 grid) {
  return a.role_gate_up ? launch_gemv_role<NB, 1>(s, a, grid) : launch_gemv_role<NB, 0>(s, a, grid);
}

// ---------------------------------------------------------------- batched projections
// More than two rows (the batch-8 and batch-32 workloads): out[b, n] =
// sum_k act[b, k] W[n, k] for b < M <= 32, act f16.  A workgroup owns
// RB = 16 RT weight rows over one K slice; its four waves split the slice
// into contiguous runs of 32-k units and meet in LDS once, at the end.  Both
// operands go straight from memory into registers (the activations are at
// most 32 rows and stay in L2): a wave issues the loads of up to MAXU units
// at once, then multiplies them, so its whole share is one memory round trip
// (the launcher sizes the slices for that) and nothing waits on a barrier
// while the weights stream.  Without a K split a workgroup is the only writer
// of its outputs: q/k/v sums are stored, residual rows read-modify-written,
// and no atomics are needed.  With one, the slices add fixed-point values
// atomically (deterministic, as above).
// In the decode step both operands are unit-tiled (qw_internal.h): a wave's
// 16-byte loads of one unit then read one contiguous 1 KB tile, where the
// row-major layout gave 16 separate 64-byte pieces per load instruction, 3 KB
// or more apart (weights) or re-read from L2 (activations).  Measured with
// the loads alone at the 32-row gate/up shape: 22.8 -> 15.0 us per launch.
template <int RT, int NB, int MAXU, DecOut OM, bool ATOMIC, int NW = 4>
__global__ void __launch_bounds__(64 * NW) dec_rows_kernel(DecGemvArgs a) {
  constexpr int RB = 16 * RT, BT = 16 * NB, NT = 64 * NW;
  static_assert(OM != DecOut::Logits || NW == 4, "the argmax partials take 256 threads");
  __shared__ float s_acc[NW][RB][BT + 1];
  __shared__ float s_part[NT / 32][32], s_rstd[32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: unit bounds stay scalar
  const int i = lane & 15, g = lane >> 4;
  const int nblk = blockIdx.x, split = blockIdx.y;
  const int n0 = nblk * RB;
  const int units = a.K >> 5;
  const int us0 = split * a.units_per_split, us1 = min(units, us0 + a.units_per_split);
  const int per_w = (max(0, us1 - us0) + NW - 1) / NW;
  const int u0 = us0 + wave * per_w, u1 = min(us1, u0 + per_w);

  if (a.clear)
    clear_share(a.clear, a.clear_n, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  // operand u without 1/rms: the row sums of squares, needed at the end
  const bool nrm = a.nin.ss != nullptr;
  RowRstd<NT> rr;
  if (nrm) rr.load(a.nin, a.M);

  // lane (i, g): weight row n0 + 16 r + i and batch row 16 nb + i, k offset 8 g
  // of each unit; rows past N or M are clamped and their results never stored
  // unit-tiled operands: a unit's 16 x 32 tile is one 1 KB piece (lane l
  // reads bytes 16 l ..), tiles of a row block 512 elements apart
  const f16 *wp[RT];
  const f16 *xp[NB];
  const int wstr = a.w_tiled ? 512 : 32, xstr = a.act_tiled ? 512 : 32;     // elements per unit
#pragma unroll
  for (int r = 0; r < RT; ++r)
    wp[r] = (const f16 *)a.W + (a.w_tiled ? (int64_t)(nblk * RT + r) * units * 512 + 8 * lane
                                          : (int64_t)min(n0 + 16 * r + i, a.N - 1) * a.K + 8 * g);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    xp[nb] = (const f16 *)a.act + (a.act_tiled ? (int64_t)nb * units * 512 + 8 * lane
                                               : (int64_t)min(16 * nb + i, a.M - 1) * a.lda + 8 * g);

  f32x4 acc[RT][NB];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[r][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ub = u0; ub < u1; ub += MAXU) {
    f16x8 w[MAXU][RT], x[MAXU][NB];
#pragma unroll
    for (int t = 0; t < MAXU; ++t) {
      if (ub + t < u1) {        // uniform (scalar) condition: no load past the share
#pragma unroll
        for (int r = 0; r < RT; ++r) w[t][r] = load8(wp[r] + (int64_t)wstr * (ub + t));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) x[t][nb] = load8(xp[nb] + (int64_t)xstr * (ub + t));
      }
    }
    // keep every load of the batch ahead of the first multiply (the
    // scheduler would otherwise wait for the first unit mid-batch)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < MAXU; ++t) {
      if (ub + t < u1) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[r][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w[t][r], x[t][nb], acc[r][nb], 0, 0, 0);
      }
    }
  }

  // lane (i, g) holds rows 4g .. 4g + 3 of tile r, batch column 16 nb + i
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) s_acc[wave][16 * r + 4 * g + q][16 * nb + i] = acc[r][nb][q];
  __syncthreads();
  if (nrm) rr.finish(a.nin, s_part, s_rstd);
  auto total = [&](int nl, int b) {
    float t = s_acc[0][nl][b];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) t += s_acc[w2][nl][b];
    return nrm ? t * a.scale * s_rstd[b] : t * a.scale;
  };

  if constexpr (OM == DecOut::FixAdd) {
    for (int e = tid; e < RB * BT; e += NT) {
      const int nl = e % RB, b = e / RB, n = n0 + nl;
      if (n >= a.N || b >= a.M) continue;
      long long *p = a.out_fix + (int64_t)b * a.ldo + n;
      if constexpr (ATOMIC) {
        fix_add(p, total(nl, b), a.num_flag);
      } else {
        // sole writer: a residual row adds to its value, a projection sum
        // (cleared beforehand) is simply its value
        *p += to_fix(total(nl, b), a.num_flag);
      }
    }
    // a residual projection hands the next RMSNorm its operand
    if (a.nout.w) norm_tail<RB, BT, NT>(a, n0, nblk, &s_acc[0][0][0]);
  } else if constexpr (OM == DecOut::SwiGLUOut) {
    static_assert(RT % 2 == 0, "gate/up rows come in GU_BLOCK pairs");
    f16 *h = (f16 *)a.h_out;
    for (int e = tid; e < (RB / 2) * BT; e += NT) {
      const int fl = e % (RB / 2), b = e / (RB / 2);
      const int p = fl / GU_BLOCK, j = fl % GU_BLOCK;
      const int f = nblk * (RB / 2) + fl;
      if (b >= a.M || f >= a.N / 2) continue;
      const float gt = total(2 * GU_BLOCK * p + j, b), up = total(2 * GU_BLOCK * p + GU_BLOCK + j, b);
      h[a.act_tiled ? tile_off(b, f, a.ldh) : (int64_t)b * a.ldh + f] = (f16)(silu_f(gt) * up);
    }
  } else {
    // logits (optional copy) and this block's (max, lowest index) per batch row
    static_assert(RB == 64, "the argmax partials are laid out per 64 vocabulary rows");
    constexpr int TPB = 256 / BT;               // threads per batch row
    const int b = tid / TPB, sub = tid % TPB;
    float best = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < RB / TPB; ++j) {
      const int nl = sub + TPB * j, n = n0 + nl;
      const float v = total(nl, b);
      if (n < a.N && b < a.M) {
        if (a.logits) a.logits[(int64_t)b * a.ldo + n] = v;
        if (v > best) { best = v; bi = n; }      // n increases with j
        if (!(fabsf(v) <= 3.4e38f)) atomicOr(a.num_flag, kFlagNonFinite);
      }
    }
#pragma unroll
    for (int off = 1; off < TPB; off <<= 1) {
      const float ob = __shfl_xor(best, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    if (sub == 0 && b < a.M) {
      a.arg_v[(int64_t)b * gridDim.x + nblk] = best;
      a.arg_i[(int64_t)b * gridDim.x + nblk] = bi;
    }
  }
}

// units a wave loads at once: at most about 200 registers of operands
template <int RT, int NB>
constexpr int rows_maxu() { return (RT + NB) * 4 * 16 <= 200 ? 16 : (RT + NB) * 4 * 12 <= 200 ? 12 : 8; }

// How a batched projection is cut: RT 16-row tiles per workgroup, NW waves
// splitting each workgroup's K slice, `splits` K slices (atomics when > 1).
// Every workgroup reads the whole activation block of its K slice from L2, and
// the per-CU path to L2 (not HBM) bounds these kernels, so more rows per
// workgroup cut the traffic that matters; more waves keep each wave's share
// within one batch of loads.
struct RowsPlan {
  int rt, nw, splits;
};

template <int NB, int RT, int NW>
hipError_t launch_rows_fix(hipStream_t s, const DecGemvArgs &a, int splits) {
  constexpr int MU = rows_maxu<RT, NB>();
  const dim3 grid((a.N + 16 * RT - 1) / (16 * RT), splits);
  if (splits > 1)
    QW_LAUNCH((dec_rows_kernel<RT, NB, MU, DecOut::FixAdd, true, NW>), dim3(grid), dim3(64 * NW), 0, s, a);
  else
    QW_LAUNCH((dec_rows_kernel<RT, NB, MU, DecOut::FixAdd, false, NW>), dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int NB, int RT, int NW>
hipError_t launch_rows_swiglu(hipStream_t s, const DecGemvArgs &a) {
  constexpr int MU = rows_maxu<RT, NB>();
  const dim3 grid((a.N + 16 * RT - 1) / (16 * RT), 1);
  QW_LAUNCH((dec_rows_kernel<RT, NB, MU, DecOut::SwiGLUOut, false, NW>), dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_rows_nb(hipStream_t s, const DecGemvArgs &a, const RowsPlan &p) {
  if (a.logits_mode) {
    const dim3 grid((a.N + 63) / 64, 1);
    QW_LAUNCH((dec_rows_kernel<4, NB, rows_maxu<4, NB>(), DecOut::Logits, false>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int key = p.rt * 10 + p.nw;
  if (a.swiglu_out) {
    switch (key) {
      case 24: return launch_rows_swiglu<NB, 2, 4>(s, a);
      case 28: return launch_rows_swiglu<NB, 2, 8>(s, a);
      case 44: return launch_rows_swiglu<NB, 4, 4>(s, a);
      case 48: return launch_rows_swiglu<NB, 4, 8>(s, a);
      default: return hipErrorInvalidValue;
    }
  }
  switch (key) {
    case 14: return launch_rows_fix<NB, 1, 4>(s, a, p.splits);
    case 18: return launch_rows_fix<NB, 1, 8>(s, a, p.splits);
    case 24: return launch_rows_fix<NB, 2, 4>(s, a, p.splits);
    case 28: return launch_rows_fix<NB, 2, 8>(s, a, p.splits);
    case 44: return launch_rows_fix<NB, 4, 4>(s, a, p.splits);
    case 48: return launch_rows_fix<NB, 4, 8>(s, a, p.splits);
    default: return hipErrorInvalidValue;
  }
}

int rows_maxu_rt(int rt, int nb) {
  switch (rt * 10 + nb) {
    case 11: return rows_maxu<1, 1>();
    case 12: return rows_maxu<1, 2>();
    case 21: return rows_maxu<2, 1>();
    case 22: return rows_maxu<2, 2>();
    case 41: return rows_maxu<4, 1>();
    default: return rows_maxu<4, 2>();
  }
}

// K slices of a split batched projection: about `target` workgroups of RT
// tiles, at least enough slices that each wave's share is one batch of loads,
// at most one unit per wave.
int rows_splits(int N, int units, int rt, int nw, int target, int nb) {
  const int blocks = (N + 16 * rt - 1) / (16 * rt);
  const int mu = rows_maxu_rt(rt, nb);
  int rs = (target + blocks / 2) / blocks;
  rs = max(rs, (units + nw * mu - 1) / (nw * mu));
  return max(1, min(rs, units / nw));
}

// The cut of each batched projection (the gate/up one is never split: its
// SwiGLU epilogue needs whole sums).  Measured at 32 rows on the 1.5B shapes
// (ms per decode step, 28 layers): the split projections with 32-row tiles,
// 8 waves and about 256 workgroups against 16-row tiles, 4 waves and about
// 512 (down 0.480 -> 0.378, o 0.201 -> 0.183, q/k/v 0.201 -> 0.185); larger
// gate/up tiles were slower (64 rows: 0.715 -> 0.76-0.78, 280 workgroups
// spread unevenly over 256 CUs).
RowsPlan rows_plan(const DecGemvArgs &a, int units) {
  const int nb = a.M <= 16 ? 1 : 2;
  RowsPlan p;
  if (a.swiglu_out) {
    p = {2, 4, 1};
  } else if (nb == 2) {
    p = {2, 8, rows_splits(a.N, units, 2, 8, 256, nb)};
  } else {
    p = {1, 4, rows_splits(a.N, units, 1, 4, 512, nb)};
  }
#ifdef QW_TUNING
  // tuning builds only: QW_ROWS_PLAN="gu=RT,NW;fix=RT,NW,TARGET" overrides the cut
  if (const char *env = getenv("QW_ROWS_PLAN")) {
    int rt, nw, tg;
    const char *gu = strstr(env, "gu="), *fx = strstr(env, "fix=");
    if (a.swiglu_out && gu && sscanf(gu, "gu=%d,%d", &rt, &nw) == 2) p = {rt, nw, 1};
    if (!a.swiglu_out && fx && sscanf(fx, "fix=%d,%d,%d", &rt, &nw, &tg) == 3)
      p = {rt, nw, rows_splits(a.N, units, rt, nw, tg, nb)};
  }
#endif
  return p;
}

// ---------------------------------------------------------------- fused MLP
// For one or two rows the MLP of a layer ("LLM Speedrun: Architecture",
// "But how does it remember things?": gated SiLU MLP) is a single kernel:
//   x_out = x_in + W_down (silu(W_gate u) * (W_up u)),  u = RMSNorm(x_in) * w.
// Workgroup p owns the GU_BLOCK intermediate features f0 = 16p .. 16p + 15.
// It forms their gate and up values over the whole hidden width (MFMA, the
// four waves split K and meet in LDS), applies SwiGLU, and multiplies the 16
// values into rows f0 .. f0 + 15 of the transposed down weight, adding the H
// results per row into x_out.  The down projection is thus split over its K
// (= I) across the workgroups and needs neither a launch nor a buffer of its
// own.  x_in and x_out are different buffers, so no workgroup reads a value
// that another one is adding to; workgroup 0 also adds x_in itself (exactly,
// in fixed point), so x_out must be zero on entry.  Every weight load of the
// workgroup is issued before the norm prologue.
constexpr int MLP_F = GU_BLOCK;

template <int NR, int KU>
__global__ void __launch_bounds__(256) dec_mlp_kernel(DecMlpArgs a) {
  constexpr int NPER = KU / 2;                  // residual values per thread (H <= 256 NPER = 128 KU)
  // normalised rows (f16) during gate/up, then the down results (fp32)
  __shared__ float s_buf[NR * 256 * NPER];
  f16 (*s_row)[256 * NPER] = reinterpret_cast<f16 (*)[256 * NPER]>(s_buf);
  __shared__ float s_red[4][NR];
  __shared__ float s_gu[4][2][NR][MLP_F];
  __shared__ float s_h[NR][MLP_F];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int p = blockIdx.x, f0 = p * MLP_F;
  const int H = a.H;
  const f16x8 zero = {};
  clear_share(a.clear, a.clear_n, p, gridDim.x);

  // gate row f0 + i and up row f0 + i (packed rows 2 f0 + i and 2 f0 + 16 + i);
  // wave w covers k in [w H / 4, (w + 1) H / 4)
  const f16 *Wg = (const f16 *)a.w_gu + (int64_t)(2 * f0 + i) * H;
  const f16 *Wu = Wg + (int64_t)GU_BLOCK * H;
  const int ku = H / 128;
  const int kw0 = wave * ku * 32;
  f16x8 wg[KU], wu[KU];
#pragma unroll
  for (int t = 0; t < KU; ++t) {
    const bool ok = t < ku;
    const int k = kw0 + 32 * t + 8 * g;
    wg[t] = ok ? load8(Wg + k) : zero;
    wu[t] = ok ? load8(Wu + k) : zero;
  }
  // down weights: rows f0 .. f0 + 15 of W_down^T, columns n .. n + 7
  const int n = 8 * tid;
  const bool n_ok = n < H;
  const f16 *Wd = (const f16 *)a.w_down_t + (int64_t)f0 * H + (n_ok ? n : 0);
  f16x8 wd[MLP_F];
#pragma unroll
  for (int f = 0; f < MLP_F; ++f) wd[f] = load8(Wd + (int64_t)f * H);     // lanes past H: never stored

  // u = RMSNorm(x_in) * w into LDS (one round trip, one block reduction);
  // x_in is the sum of its replicas (exact, in fixed point)
  long long xq[NR][NPER];
  {
    float xv[NR][NPER], wv[NPER];
    long long qr[kXReps][NR][NPER];
#pragma unroll
    for (int t = 0; t < NPER; ++t) {
      const int c = t * 256 + tid, cc = min(c, H - 1);
      const float w = a.norm_w[cc];
      wv[t] = c < H ? w : 0.f;
#pragma unroll
      for (int r = 0; r < kXReps; ++r)
#pragma unroll
        for (int b = 0; b < NR; ++b) {
          const long long v = a.x_in[r * a.rep_stride + (int64_t)b * H + cc];
          qr[r][b][t] = c < H ? v : 0;
        }
    }
#pragma unroll
    for (int t = 0; t < NPER; ++t)
#pragma unroll
      for (int b = 0; b < NR; ++b) {
        xq[b][t] = qr[0][b][t];
#pragma unroll
        for (int r = 1; r < kXReps; ++r) xq[b][t] += qr[r][b][t];
      }
#pragma unroll
    for (int t = 0; t < NPER; ++t)
#pragma unroll
      for (int b = 0; b < NR; ++b) xv[b][t] = from_fix(xq[b][t]);
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < NPER; ++t) ss += xv[b][t] * xv[b][t];
      ss = wave_sum(ss);
      if (lane == 0) s_red[wave][b] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      const float inv = 1.0f / sqrtf((s_red[0][b] + s_red[1][b] + s_red[2][b] + s_red[3][b]) / (float)H + a.eps);
#pragma unroll
      for (int t = 0; t < NPER; ++t) {
        const int c = t * 256 + tid;
        if (c < H) s_row[b][c] = (f16)(xv[b][t] * inv * wv[t]);
      }
    }
    __syncthreads();
  }

  // gate and up sums of this wave's K quarter: lane (i, g) gets features
  // f0 + 4g .. f0 + 4g + 3 of row i
  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < KU; ++t) {
    if (t < ku) {
      const f16x8 xl = *reinterpret_cast<const f16x8 *>(&s_row[i < NR ? i : 0][kw0 + 32 * t + 8 * g]);
      const f16x8 x = (i < NR) ? xl : zero;
      ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(wg[t], x, ag, 0, 0, 0);
      au = __builtin_amdgcn_mfma_f32_16x16x32_f16(wu[t], x, au, 0, 0, 0);
    }
  }
  if (i < NR) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s_gu[wave][0][i][4 * g + r] = ag[r];
      s_gu[wave][1][i][4 * g + r] = au[r];
    }
  }
  __syncthreads();
  if (tid < NR * MLP_F) {
    const int b = tid / MLP_F, f = tid % MLP_F;
    const float gt = (s_gu[0][0][b][f] + s_gu[1][0][b][f] + s_gu[2][0][b][f] + s_gu[3][0][b][f]) * a.gu_scale;
    const float up = (s_gu[0][1][b][f] + s_gu[1][1][b][f] + s_gu[2][1][b][f] + s_gu[3][1][b][f]) * a.gu_scale;
    s_h[b][f] = silu_f(gt) * up;
  }
  __syncthreads();

  // down: y[b][n .. n + 7] = sum_f h[b][f] * W_down^T[f0 + f][n .. n + 7] into
  // LDS (reusing the normalised rows' space), then one atomic per value with
  // consecutive lanes on consecutive addresses
  float *s_y = s_buf;                                       // [NR][H], H <= 2048
  __syncthreads();                                          // the MFMA reads of s_row are done
  if (n_ok) {
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < MLP_F; ++f) {
        const float hf = s_h[b][f];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fmaf(hf, (float)wd[f][e], y[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s_y[b * H + n + e] = y[e] * a.down_scale;
    }
  }
  __syncthreads();
  // workgroups start their adds at different 64-column blocks (rotating by
  // p), so the atomics arriving at one address at a time come from few
  // workgroups; workgroup 0 starts at column 0, where its xq values line up
  long long *xo = a.x_out + (p % kXReps) * a.rep_stride;
  const int rot = 64 * (p % (H / 64));
#pragma unroll
  for (int b = 0; b < NR; ++b)
#pragma unroll
    for (int t = 0; t < NPER; ++t) {
      const int cl = t * 256 + tid;
      if (cl < H) {
        const int c = (cl + rot) % H;
        const long long v = to_fix(s_y[b * H + c], a.num_flag) + (p == 0 ? xq[b][t] : 0);
        atomicAdd(reinterpret_cast<unsigned long long *>(xo + (int64_t)b * H + c), (unsigned long long)v);
      }
    }
}

// ---------------------------------------------------------------- attention
// grid (split, kv head j, sequence b), 256 threads.  Prologue: the group's g
// query heads and the new k and v from the fixed-point q/k/v sums + bias,
// RoPE at `pos` (q rounded to f16 like the prefill path); the split that
// holds position pos writes k and v into the cache.  Body: the split's cached
// keys, plus key pos from LDS; HD/8 lanes share one key (16 bytes each);
// online softmax in the exp2 domain.  Two wave layouts:
//   WH == G  (key-parallel): every wave carries all g heads over a quarter of
//            the keys; the four waves are merged in LDS at the end.
//   WH <  G  (head-parallel): wave w carries heads w*WH .. w*WH+WH-1 over all
//            keys, so each lane's chain is WH heads long and no cross-wave
//            merge is needed (short contexts, where latency dominates).
// With one split the normalised output is written (f16); otherwise the
// split's (max, sum, unnormalised output) per head go to the partials that
// the o projection merges.
template <int HD, int G, int WH>
__global__ void __launch_bounds__(256) dec_attn_kernel(DecAttnArgs a) {
  constexpr int NW = 4;
  constexpr bool KEYPAR = (WH == G);
  constexpr int LPK = HD / 8;        // lanes per key
  constexpr int KPW = 64 / LPK;      // keys per wave per load
  constexpr int KSTEP = KEYPAR ? NW * KPW : KPW;   // keys between a wave's consecutive loads
  constexpr int HALF = HD / 2;
  __shared__ float s_q[G][HD];
  __shared__ float s_k[HD], s_v[HD];
  __shared__ float s_m[KEYPAR ? NW : 1][G], s_l[KEYPAR ? NW : 1][G];
  __shared__ float s_o[KEYPAR ? NW : 1][G][HD];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slot = lane / LPK, dl = lane % LPK, d0 = dl * 8;
  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int S = gridDim.x;
  const int pos = a.pos_dev[b];
  const int n_keys = pos + 1;
  int per = (n_keys + S - 1) / S;
  per = (per + NW * KPW - 1) / (NW * KPW) * (NW * KPW);
  const int kb0 = split * per;
  const int kb1 = min(n_keys, kb0 + per);
  const bool has_new = kb0 <= pos && pos < kb1;

  // the heads this wave carries: h_lo + t for t < nh
  const int h_lo = KEYPAR ? 0 : wave * WH;
  const int nh = KEYPAR ? G : max(0, min(WH, G - h_lo));
  f16 *Kc = (f16 *)a.k_cache;
  f16 *Vc = (f16 *)a.v_cache;

  // cached keys of this split, U loads per lane in flight: the first batch
  // goes out before the prologue (it does not depend on it), each next batch
  // before the current one is consumed
  constexpr int U = 4;
  const int kc_end = min(kb1, pos);
  const int kstart = kb0 + (KEYPAR ? wave * KPW : 0);
  f16x8 kr[U], vr[U];
  auto issue = [&](int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = kb + u * KSTEP + slot;
      // out-of-range keys get weight 0; their values must be finite
      const int tc = min(t, max(kc_end - 1, 0));
      const int64_t off = kv_offset(a.kv, a.n_kv_heads, HD, b, j, tc) + d0;
      const f16x8 kv = load8(Kc + off), vv = load8(Vc + off);
      kr[u] = t < kc_end ? kv : f16x8{};
      vr[u] = t < kc_end ? vv : f16x8{};
    }
  };
  if (nh > 0 && kstart < kc_end) issue(kstart);

  const int nq = a.n_kv_heads * G;
  const int qd = nq * HD, kvd = a.n_kv_heads * HD;
  const int ncols = qd + 2 * kvd;
  const long long *acc = a.qkv_fix + (int64_t)b * ncols;
  const float2 *cs = a.rope + (int64_t)pos * HALF;
  const float qscale = a.softmax_scale * LOG2E;

  // side job: clear the gate/up accumulator (its last reader finished)
  clear_share(a.clear, a.clear_n, (b * gridDim.y + j) * S + split, S * gridDim.y * gridDim.z);

  for (int e = tid; e < (G + 1) * HALF + HD; e += 256) {
    if (e < (G + 1) * HALF) {
      const int hh = e / HALF, i = e % HALF;
      const int c0 = (hh < G) ? (j * G + hh) * HD + i : qd + j * HD + i;
      const float re = from_fix(acc[c0]) + a.bias[c0];
      const float im = from_fix(acc[c0 + HALF]) + a.bias[c0 + HALF];
      const float2 r = cs[i];
      const float nre = re * r.x - im * r.y, nim = im * r.x + re * r.y;
      if (hh < G) {
        s_q[hh][i] = (float)(f16)nre * qscale;
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
  if (has_new && tid < HD) {
    const int64_t np = kv_offset(a.kv, a.n_kv_heads, HD, b, j, pos);
    Kc[np + tid] = (f16)s_k[tid];
    Vc[np + tid] = (f16)s_v[tid];
  }

  float q[WH][8];
#pragma unroll
  for (int t = 0; t < WH; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[t][e] = (t < nh) ? s_q[h_lo + t][d0 + e] : 0.f;
  float m[WH], l[WH], o[WH][8];
#pragma unroll
  for (int t = 0; t < WH; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[t][e] = 0.f;
  }

  auto visit = [&](const float *kf, const float *vf) {
#pragma unroll
    for (int t = 0; t < WH; ++t) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(q[t][e], kf[e], s);
      s = group_sum<LPK>(s);
      const float mn = fmaxf(m[t], s);
      const float corr = exp2f(m[t] - mn);
      const float p = exp2f(s - mn);
      l[t] = l[t] * corr + p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[t][e] = fmaf(p, vf[e], o[t][e] * corr);
      m[t] = mn;
    }
  };

  if (nh > 0) {
    for (int kb = kstart; kb < kc_end; kb += U * KSTEP) {
      f16x8 kc[U], vc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kc[u] = kr[u];
        vc[u] = vr[u];
      }
      if (kb + U * KSTEP < kc_end) issue(kb + U * KSTEP);
      // the U keys of this lane at once: one running-max update and one
      // rescale per batch instead of per key
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) ok[u] = kb + u * KSTEP + slot < kc_end;
#pragma unroll
      for (int t = 0; t < WH; ++t) {
        float sc[U];
        float mx = m[t];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(q[t][e], (float)kc[u][e], d);
          d = group_sum<LPK>(d);
          sc[u] = ok[u] ? d : -INFINITY;
          mx = fmaxf(mx, sc[u]);
        }
        const float corr = (m[t] == -INFINITY) ? 0.f : exp2f(m[t] - mx);
        float lsum = 0.f;
        float acc8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc8[e] = o[t][e] * corr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = (mx == -INFINITY) ? 0.f : exp2f(sc[u] - mx);
          lsum += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc8[e] = fmaf(p, (float)vc[u][e], acc8[e]);
        }
        l[t] = l[t] * corr + lsum;
        m[t] = mx;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[t][e] = acc8[e];
      }
    }
    if (has_new && (KEYPAR ? wave == 0 : true) && slot == 0) {
      float kf[8], vf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { kf[e] = s_k[d0 + e]; vf[e] = s_v[d0 + e]; }
      visit(kf, vf);
    }
  }

  // merge the KPW key slots of each wave (lanes with equal dl)
#pragma unroll
  for (int t = 0; t < WH; ++t) {
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m[t], off, 64);
      const float lo = __shfl_xor(l[t], off, 64);
      const float mn = fmaxf(m[t], mo);
      const float ca = (m[t] == -INFINITY) ? 0.f : exp2f(m[t] - mn);
      const float cb = (mo == -INFINITY) ? 0.f : exp2f(mo - mn);
      l[t] = l[t] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float oo = __shfl_xor(o[t][e], off, 64);
        o[t][e] = o[t][e] * ca + oo * cb;
      }
      m[t] = mn;
    }
  }

  if constexpr (!KEYPAR) {
    // each wave owns its heads: write them directly (lanes of slot 0)
    if (slot == 0) {
#pragma unroll
      for (int t = 0; t < WH; ++t) {
        if (t >= nh) continue;
        const int h = j * G + h_lo + t;
        if (S == 1) {
          const float inv = 1.0f / l[t];
          f16 *out = (f16 *)a.o + (a.o_tiled ? tile_off(b, h * HD + d0, qd) : (int64_t)b * qd + h * HD + d0);
#pragma unroll
          for (int e = 0; e < 8; ++e) out[e] = (f16)(o[t][e] * inv);
        } else {
          const int64_t st = ((int64_t)b * nq + h) * S + split;
          if (dl == 0) {
            a.part_m[st] = m[t];
            a.part_l[st] = l[t];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) a.part_o[st * HD + d0 + e] = o[t][e];
        }
      }
    }
    return;
  } else {
    if (slot == 0) {
#pragma unroll
      for (int t = 0; t < WH; ++t) {
        if (dl == 0) {
          s_m[wave][t] = m[t];
          s_l[wave][t] = l[t];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s_o[wave][t][d0 + e] = o[t][e];
      }
    }
    __syncthreads();
    for (int e = tid; e < G * HD; e += 256) {
      const int hh = e / HD, d = e % HD;
      float M = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, s_m[w2][hh]);
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
          const float c = (s_m[w2][hh] == -INFINITY) ? 0.f : exp2f(s_m[w2][hh] - M);
          L += s_l[w2][hh] * c;
          O += s_o[w2][hh][d] * c;
        }
      }
      const int h = j * G + hh;
      if (S == 1) {
        ((f16 *)a.o)[a.o_tiled ? tile_off(b, h * HD + d, qd) : (int64_t)b * qd + h * HD + d] = (f16)(O / L);
      } else {
        const int64_t st = ((int64_t)b * nq + h) * S + split;
        if (d == 0) {
          a.part_m[st] = M;
          a.part_l[st] = L;
        }
        a.part_o[st * HD + d] = O;
      }
    }
  }
}

// Split-KV decode attention on the matrix cores, for batches of more than two
// rows (grid: split x KV head x row).  The g query heads of the KV group are
// the columns of the MFMA B operand (g <= 8 of 16 used):
//   S^T  = K . Q^T    A = 16 keys x 32 dims, 16-byte loads from the cache rows
//   O^T += V^T . P^T  A = 16 dims x 32 keys, gathered 2 bytes at a time from
//                     the cache rows (each element is still read once)
// Within a 32-key chunk the key rows are visited in the order that makes the
// 8 probabilities a lane holds 8 consecutive keys, which is the B operand of
// the second product as it stands.  Wave w takes chunks w, w + 4, ...; the
// four waves' (max, sum, output) meet in LDS.  Prologue, cache write, the new
// key (from LDS) and the partials are those of dec_attn_kernel.
template <int HD, int G>
__global__ void __launch_bounds__(256) dec_attn_mfma_kernel(DecAttnArgs a) {
  constexpr int NW = 4, HALF = HD / 2, KS = HD / 32, DT = HD / 16;
  static_assert(G <= 16, "heads of a group fit the 16 MFMA columns");
  __shared__ float s_q[G][HD];
  __shared__ float s_k[HD], s_v[HD];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_o[NW][G][HD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int S = gridDim.x;
  const int pos = a.pos_dev[b];
  const int n_keys = pos + 1;
  int per = (n_keys + S - 1) / S;
  per = (per + 31) / 32 * 32;
  const int kb0 = split * per;
  const int kb1 = min(n_keys, kb0 + per);
  const bool has_new = kb0 <= pos && pos < kb1;
  const int nq = a.n_kv_heads * G;
  const int qd = nq * HD, kvd = a.n_kv_heads * HD;
  const int ncols = qd + 2 * kvd;
  const long long *acc = a.qkv_fix + (int64_t)b * ncols;
  const float2 *cs = a.rope + (int64_t)pos * HALF;
  f16 *Kc = (f16 *)a.k_cache;
  f16 *Vc = (f16 *)a.v_cache;

  // the wave's first batch of cached keys is loaded before the prologue, so
  // that it arrives while bias + RoPE run; later batches at the end of each
  // step.  Keys past the split's end load a clamped (valid) row.
  const int kc_end = min(kb1, pos);             // cached keys of this split
  const int klast = max(kc_end - 1, 0);
  // A batch is 32 keys from a multiple of 32 (clamped to klast), so it lies in
  // one cache block: its rows are addressed from the block's first position.
  auto batch_base = [&](int k0) -> int64_t {
    return kv_offset(a.kv, a.n_kv_heads, HD, b, j, min(k0, klast) & ~(kKvBlock - 1));
  };
  // K rows of the two 16-key tiles: tile y, row i is key k0 + 8 (i / 4) + 4y + i % 4;
  // V^T operand: lane (i, g) holds dim 16d + i of keys k0 + 8g .. k0 + 8g + 7
  f16x8 kf[2][KS], vf[DT];
  auto load_kv = [&](int k0, int64_t base) {
    const int kb = min(k0, klast) & ~(kKvBlock - 1);
    const f16 *Kb = Kc + base, *Vb = Vc + base;
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int key = min(k0 + 8 * (i >> 2) + 4 * y + (i & 3), klast) - kb;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) kf[y][s2] = load8(Kb + (int64_t)key * HD + 32 * s2 + 8 * g);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f16 *vrow = Vb + (int64_t)(min(k0 + 8 * g + e, klast) - kb) * HD + i;
#pragma unroll
      for (int d = 0; d < DT; ++d) vf[d][e] = vrow[16 * d];
    }
  };
  // prologue operands (q of the group's heads, new k and v: projection sums,
  // biases, the rotation at pos) are loaded first, then the first key batch,
  // so that bias + RoPE waits only for its own loads.  Element e < (G+1) HALF
  // is a rotation pair of q (head e / HALF) or k, the rest one value of v;
  // addresses of unused elements are clamped and their values discarded.
  constexpr int NE = (G + 1) * HALF + HD, NI = (NE + 255) / 256;
  long long pa0[NI], pa1[NI];
  float pb0[NI], pb1[NI];
  float2 pr[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int e = tid + 256 * it;
    const bool rot = e < (G + 1) * HALF, val = e < NE;
    const int hh = rot ? e / HALF : 0, ii = rot ? e % HALF : 0;
    const int c0 = rot ? ((hh < G) ? (j * G + hh) * HD + ii : qd + j * HD + ii)
                       : qd + kvd + j * HD + (val ? e - (G + 1) * HALF : 0);
    const int c1 = rot ? c0 + HALF : c0;
    pa0[it] = acc[c0];
    pa1[it] = acc[c1];
    pb0[it] = a.bias[c0];
    pb1[it] = a.bias[c1];
    pr[it] = cs[ii];
  }
  __builtin_amdgcn_sched_barrier(0);
  const int kfirst = kb0 + 32 * wave;
  load_kv(kfirst, batch_base(kfirst));
  __builtin_amdgcn_sched_barrier(0);

  clear_share(a.clear, a.clear_n, (b * gridDim.y + j) * S + split, S * gridDim.y * gridDim.z);

  // q of the group's heads (rounded to f16, unscaled), new k and v
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int e = tid + 256 * it;
    if (e < (G + 1) * HALF) {
      const int hh = e / HALF, ii = e % HALF;
      const float re = from_fix(pa0[it]) + pb0[it], im = from_fix(pa1[it]) + pb1[it];
      const float2 r = pr[it];
      const float nre = re * r.x - im * r.y, nim = im * r.x + re * r.y;
      if (hh < G) {
        s_q[hh][ii] = (float)(f16)nre;
        s_q[hh][ii + HALF] = (float)(f16)nim;
      } else {
        s_k[ii] = (float)(f16)nre;
        s_k[ii + HALF] = (float)(f16)nim;
      }
    } else if (e < NE) {
      s_v[e - (G + 1) * HALF] = (float)(f16)(from_fix(pa0[it]) + pb0[it]);
    }
  }
  lds_barrier();                   // the first key batch stays in flight
  if (has_new && tid < HD) {
    const int64_t np = kv_offset(a.kv, a.n_kv_heads, HD, b, j, pos);
    Kc[np + tid] = (f16)s_k[tid];
    Vc[np + tid] = (f16)s_v[tid];
  }

  f16x8 qf[KS];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[s2][e] = (i < G) ? (f16)s_q[i < G ? i : 0][32 * s2 + 8 * g + e] : (f16)0.f;
  const float sl2 = a.softmax_scale * LOG2E;
  float m = -INFINITY, l = 0.f;                 // head i
  f32x4 o[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kfirst; k0 < kc_end; k0 += 32 * NW) {
    // the next batch's block, looked up while this batch is multiplied
    const int64_t next_base = batch_base(k0 + 32 * NW);
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) sacc[y] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[y][s2], qf[s2], sacc[y], 0, 0, 0);
    // lane (i, g) now holds head i's scores of keys k0 + 8g + 4y + r
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = (k0 + 8 * g + 4 * y + r < kc_end) ? sacc[y][r] * sl2 : -INFINITY;
        sc[4 * y + r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);             // finite: key k0 is in range
    const float corr = exp2f(m - mn);
    float sum = 0.f;
    f16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = exp2f(sc[e] - mn);
      sum += p;
      pb[e] = (f16)p;
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    l = l * corr + sum;
    m = mn;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      o[d] *= corr;
      o[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[d], pb, o[d], 0, 0, 0);
    }
    if (k0 + 32 * NW < kc_end) load_kv(k0 + 32 * NW, next_base);
  }
  if (has_new && wave == 0) {
    // the new key, from LDS: head i's score, then its share of dims 16d + 4g + r
    float dsum = 0.f;
#pragma unroll 8
    for (int e = 0; e < HD; ++e) dsum = fmaf(s_q[i < G ? i : 0][e], s_k[e], dsum);
    const float sc = dsum * sl2;
    const float mn = fmaxf(m, sc);
    const float corr = exp2f(m - mn);
    const float p = exp2f(sc - mn);
    l = l * corr + p;
    m = mn;
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[d][r] = o[d][r] * corr + p * s_v[16 * d + 4 * g + r];
  }

  if (i < G) {
    if (g == 0) {
      s_m[wave][i] = m;
      s_l[wave][i] = l;
    }
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[wave][i][16 * d + 4 * g + r] = o[d][r];
  }
  __syncthreads();
  for (int e = tid; e < G * HD; e += 256) {
    const int hh = e / HD, d = e % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, s_m[w2][hh]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        const float c = (s_m[w2][hh] == -INFINITY) ? 0.f : exp2f(s_m[w2][hh] - M);
        L += s_l[w2][hh] * c;
        O += s_o[w2][hh][d] * c;
      }
    }
    const int h = j * G + hh;
    if (S == 1) {
      ((f16 *)a.o)[a.o_tiled ? tile_off(b, h * HD + d, qd) : (int64_t)b * qd + h * HD + d] = (f16)(O / L);
    } else {
      const int64_t st = ((int64_t)b * nq + h) * S + split;
      if (d == 0) {
        a.part_m[st] = M;
        a.part_l[st] = L;
      }
      a.part_o[st * HD + d] = O;
    }
  }
}

constexpr bool kMfmaDecodeAttn = true;

template <int HD, int G>
hipError_t launch_attn_g(hipStream_t s, const DecAttnArgs &a, dim3 grid) {
  if constexpr (HD >= 64) {
    if (kMfmaDecodeAttn) {
      QW_LAUNCH((dec_attn_mfma_kernel<HD, G>), dim3(grid), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.head_parallel && G > 1) {
    QW_LAUNCH((dec_attn_kernel<HD, G, (G + 3) / 4>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  QW_LAUNCH((dec_attn_kernel<HD, G, G>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_attn_hd(hipStream_t s, const DecAttnArgs &a, dim3 grid, int g) {
  switch (g) {
    case 1: return launch_attn_g<HD, 1>(s, a, grid);
    case 2: return launch_attn_g<HD, 2>(s, a, grid);
    case 3: return launch_attn_g<HD, 3>(s, a, grid);
    case 4: return launch_attn_g<HD, 4>(s, a, grid);
    case 5: return launch_attn_g<HD, 5>(s, a, grid);
    case 6: return launch_attn_g<HD, 6>(s, a, grid);
    case 7: return launch_attn_g<HD, 7>(s, a, grid);
    case 8: return launch_attn_g<HD, 8>(s, a, grid);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// The same MLP with 32 features per workgroup and 8 waves: half the
// workgroups, so half the atomics, and workgroups light enough to all be
// resident.  Wave w multiplies tile w % 4 of the 64 packed rows (gate 0..15,
// up 0..15, gate 16..31, up 16..31) over K half w / 4; the down product is
// split over RG row groups of DR rows that meet in LDS.
// LD (late down): the down-projection weights are loaded only after the
// gate/up products, so their registers reuse the gate/up weights' and two
// workgroups fit on a CU (at 1.5B the 280 workgroups then run in one round
// instead of 256 + 24).
template <int NR, int KU, int DR, bool LD = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(LD ? 4 : 1)))
dec_mlp32_kernel(DecMlpArgs a) {
  constexpr int F = 2 * GU_BLOCK;               // features per workgroup
  constexpr int RG = F / DR;                    // row groups of the down product
  constexpr int NPER = 4;                       // residual values per thread (H <= 2048)
  constexpr int YH = 4096 / RG;                 // s_y columns per (group, row) slot: RG * YH = 4096
  __shared__ float s_buf[NR * 1024];            // normalised rows (f16, H <= 2048)
  f16 (*s_row)[2048] = reinterpret_cast<f16 (*)[2048]>(s_buf);
  __shared__ float s_red[8][NR];
  __shared__ float s_gu[8][NR][16];
  __shared__ float s_h[NR][F];
  __shared__ float s_y[RG][NR][YH];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int p = blockIdx.x, f0 = p * F;
  const int H = a.H;
  const f16x8 zero = {};
  clear_share(a.clear, a.clear_n, p, gridDim.x);

  // the residual rows and the norm weight first, so that the norm can run
  // while the weights are still arriving; then every weight of the workgroup
  float wv[NPER];
  long long qr[kXReps][NR][NPER];
#pragma unroll
  for (int t = 0; t < NPER; ++t) {
    const int c = t * 512 + tid, cc = min(c, H - 1);
    const float w = a.norm_w[cc];
    wv[t] = c < H ? w : 0.f;
#pragma unroll
    for (int r = 0; r < kXReps; ++r)
#pragma unroll
      for (int b = 0; b < NR; ++b) {
        const long long v = a.x_in[r * a.rep_stride + (int64_t)b * H + cc];
        qr[r][b][t] = c < H ? v : 0;
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int tau = wave & 3, kh = wave >> 2;
  const f16 *Wt = (const f16 *)a.w_gu + (int64_t)(2 * f0 + 16 * tau + i) * H;
  const int ku = H / 64;
  const int kw0 = kh * ku * 32;
  // unit-tiled copy: the wave's 16 rows are row block 2 f0 / 16 + tau
  const f16 *Wtl = a.w_gu_tiled ? (const f16 *)a.w_gu_tiled + ((int64_t)(2 * f0 / 16 + tau) * (H >> 5) + (kw0 >> 5)) * 512 + 8 * lane
                                : nullptr;
  f16x8 wt[KU];
  // units past ku load a clamped (in-range) address and are never multiplied:
  // a condition around the load would become a branch per load
#pragma unroll
  for (int t = 0; t < KU; ++t)
    wt[t] = Wtl ? load8(Wtl + (int64_t)min(t, ku - 1) * 512) : load8(Wt + kw0 + 32 * min(t, ku - 1) + 8 * g);
  const int CB = H / 8;
  const int rg = tid / CB, cb = tid % CB;
  const bool d_ok = rg < RG;
  const f16 *Wd = (const f16 *)a.w_down_t + (int64_t)(f0 + (d_ok ? rg : 0) * DR) * H + 8 * cb;
  f16x8 wd[DR];
  if constexpr (!LD) {
#pragma unroll
    for (int f = 0; f < DR; ++f) wd[f] = load8(Wd + (int64_t)f * H);     // threads past RG: unused
  }
  __builtin_amdgcn_sched_barrier(0);

  long long xq[NR][NPER];
  {
    float xv[NR][NPER];
#pragma unroll
    for (int t = 0; t < NPER; ++t)
#pragma unroll
      for (int b = 0; b < NR; ++b) {
        xq[b][t] = qr[0][b][t];
#pragma unroll
        for (int r = 1; r < kXReps; ++r) xq[b][t] += qr[r][b][t];
        xv[b][t] = from_fix(xq[b][t]);
      }
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < NPER; ++t) ss += xv[b][t] * xv[b][t];
      ss = wave_sum(ss);
      if (lane == 0) s_red[wave][b] = ss;
    }
    lds_barrier();                 // the weights stay in flight
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) tot += s_red[w][b];
      const float inv = 1.0f / sqrtf(tot / (float)H + a.eps);
#pragma unroll
      for (int t = 0; t < NPER; ++t) {
        const int c = t * 512 + tid;
        if (c < H) s_row[b][c] = (f16)(xv[b][t] * inv * wv[t]);
      }
    }
    lds_barrier();
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < KU; ++t) {
    if (t < ku) {
      const f16x8 xl = *reinterpret_cast<const f16x8 *>(&s_row[i < NR ? i : 0][kw0 + 32 * t + 8 * g]);
      const f16x8 x = (i < NR) ? xl : zero;
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wt[t], x, acc, 0, 0, 0);
    }
  }
  if constexpr (LD) {
#pragma unroll
    for (int f = 0; f < DR; ++f) wd[f] = load8(Wd + (int64_t)f * H);     // threads past RG: unused
  }
  if (i < NR) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s_gu[wave][i][4 * g + r] = acc[r];
  }
  __syncthreads();
  if (tid < NR * F) {
    const int b = tid / F, f = tid % F, hf = f / 16, w16 = f % 16;
    const float gt = (s_gu[2 * hf][b][w16] + s_gu[4 + 2 * hf][b][w16]) * a.gu_scale;
    const float up = (s_gu[2 * hf + 1][b][w16] + s_gu[5 + 2 * hf][b][w16]) * a.gu_scale;
    s_h[b][f] = silu_f(gt) * up;
  }
  __syncthreads();
  if (d_ok) {
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < DR; ++f) {
        const float hf = s_h[b][rg * DR + f];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fmaf(hf, (float)wd[f][e], y[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s_y[rg][b][8 * cb + e] = y[e];
    }
  }
  __syncthreads();
  long long *xo = a.x_out + (p % kXReps) * a.rep_stride;
  const int rot = 64 * (p % (H / 64));
#pragma unroll
  for (int b = 0; b < NR; ++b)
#pragma unroll
    for (int t = 0; t < NPER; ++t) {
      const int cl = t * 512 + tid;
      if (cl < H) {
        const int c = (cl + rot) % H;
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) v += s_y[r][b][c];
        long long xin = 0;
        if constexpr (LD) {
          // workgroup 0 adds the input residual (rot = 0 there, so c = cl);
          // re-read rather than kept live through the kernel
          if (p == 0)
            for (int r = 0; r < kXReps; ++r) xin += a.x_in[r * a.rep_stride + (int64_t)b * H + c];
        } else {
          xin = (p == 0) ? xq[b][t] : 0;
        }
        const long long q = to_fix(v * a.down_scale, a.num_flag) + xin;
        atomicAdd(reinterpret_cast<unsigned long long *>(xo + (int64_t)b * H + c), (unsigned long long)q);
      }
    }
}

// One row, 16 features per workgroup and 4 waves, every weight of the
// workgroup requested at the start: the gate/up rows into registers (wave w
// multiplies tile w % 2 -- gate 0..15 or up 0..15 -- over K half w / 2), the
// 16 rows of W_down^T straight into LDS (dynamic, 32 H bytes, so three
// workgroups share a CU and all I / 16 are resident at once).  The late-down
// kernel above loads the down rows only after the gate/up products, a second
// dependent round trip.
template <int KU>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
dec_mlp16_kernel(DecMlpArgs a) {
  constexpr int F = GU_BLOCK;                   // features per workgroup
  constexpr int NPER = 8;                       // residual values per thread (H <= 2048)
  extern __shared__ f16x8 s_wd[];               // W_down^T rows f0 .. f0 + F - 1, [F][H / 8]
  __shared__ f16 s_row[2048];                   // the normalised row
  __shared__ float s_red[4];
  __shared__ float s_gu[4][16];
  __shared__ float s_h[F];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int p = blockIdx.x, f0 = p * F;
  const int H = a.H;
  const f16x8 zero = {};
  clear_share(a.clear, a.clear_n, p, gridDim.x);

  // the residual row and the norm weight first, then the gate/up rows
  float wv[NPER];
  long long qr[kXReps][NPER];
#pragma unroll
  for (int t = 0; t < NPER; ++t) {
    const int c = t * 256 + tid, cc = min(c, H - 1);
    const float w = a.norm_w[cc];
    wv[t] = c < H ? w : 0.f;
#pragma unroll
    for (int r = 0; r < kXReps; ++r) {
      const long long v = a.x_in[r * a.rep_stride + cc];
      qr[r][t] = c < H ? v : 0;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int tau = wave & 1, kh = wave >> 1;
  const f16 *Wt = (const f16 *)a.w_gu + (int64_t)(2 * f0 + 16 * tau + i) * H;
  const int ku = H / 64;
  const int kw0 = kh * ku * 32;
  // unit-tiled copy: the wave's 16 rows are row block 2 f0 / 16 + tau
  const f16 *Wtl = a.w_gu_tiled ? (const f16 *)a.w_gu_tiled + ((int64_t)(2 * f0 / 16 + tau) * (H >> 5) + (kw0 >> 5)) * 512 + 8 * lane
                                : nullptr;
  f16x8 wt[KU];
#pragma unroll
  for (int t = 0; t < KU; ++t)
    wt[t] = Wtl ? load8(Wtl + (int64_t)min(t, ku - 1) * 512) : load8(Wt + kw0 + 32 * min(t, ku - 1) + 8 * g);
  __builtin_amdgcn_sched_barrier(0);

  // the norm (the weights stay in flight)
  float xv[NPER];
  {
    float ss = 0.f;
#pragma unroll
    for (int t = 0; t < NPER; ++t) {
      long long q = qr[0][t];
#pragma unroll
      for (int r = 1; r < kXReps; ++r) q += qr[r][t];
      xv[t] = from_fix(q);
      ss += xv[t] * xv[t];
    }
    ss = wave_sum(ss);
    if (lane == 0) s_red[wave] = ss;
    lds_barrier();
    const float inv = 1.0f / sqrtf((s_red[0] + s_red[1] + s_red[2] + s_red[3]) / (float)H + a.eps);
#pragma unroll
    for (int t = 0; t < NPER; ++t) {
      const int c = t * 256 + tid;
      if (c < H) s_row[c] = (f16)(xv[t] * inv * wv[t]);
    }
  }
  // the down rows: F * H / 8 16-byte chunks, 64 per load instruction, H / 128
  // instructions per wave (contiguous rows of W_down^T)
  {
    const f16 *Wd = (const f16 *)a.w_down_t + (int64_t)f0 * H;
    const int per_wave = H / 128;
    for (int q = 0; q < per_wave; ++q) {
      const int n = wave * per_wave + q;
      dma16(Wd + (int64_t)(64 * n + lane) * 8, &s_wd[64 * n]);
    }
  }
  lds_barrier();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < KU; ++t) {
    if (t < ku) {
      const f16x8 xl = *reinterpret_cast<const f16x8 *>(&s_row[kw0 + 32 * t + 8 * g]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wt[t], i == 0 ? xl : zero, acc, 0, 0, 0);
    }
  }
  if (i == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s_gu[wave][4 * g + r] = acc[r];
  }
  wait_vmcnt<0>();                 // this wave's down rows are in LDS
  __syncthreads();
  if (tid < F) {
    const float gt = (s_gu[0][tid] + s_gu[2][tid]) * a.gu_scale;
    const float up = (s_gu[1][tid] + s_gu[3][tid]) * a.gu_scale;
    s_h[tid] = silu_f(gt) * up;
  }
  __syncthreads();
  // y[c] = sum_f h[f] W_down^T[f][c]: thread cb takes columns 8 cb .. 8 cb + 7
  // (16-byte LDS reads), then y goes through LDS (over the down rows, read by
  // then) so that a wave's atomic adds cover consecutive addresses: with 8
  // columns per lane one add instruction touched 64 lines (1.5B MLP 0.81 ->
  // 1.86 ms per step)
  const int CB = H / 8;
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (tid < CB) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const float hf = s_h[f];
      const f16x8 w = s_wd[f * CB + tid];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = fmaf(hf, (float)w[e], y[e]);
    }
  }
  __syncthreads();                 // every wave is done with the down rows
  float *s_y = reinterpret_cast<float *>(s_wd);
  if (tid < CB) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_y[8 * tid + e] = y[e];
  }
  __syncthreads();
  long long *xo = a.x_out + (p % kXReps) * a.rep_stride;
  const int rot = 64 * (p % (H / 64));           // the adds start at a different column block per workgroup
  for (int cl = tid; cl < H; cl += 256) {
    const int c = (cl + rot) % H;
    long long xin = 0;
    if (p == 0)                    // workgroup 0 also adds the input residual (rot = 0 there)
      for (int r = 0; r < kXReps; ++r) xin += a.x_in[r * a.rep_stride + c];
    const long long q = to_fix(s_y[c] * a.down_scale, a.num_flag) + xin;
    atomicAdd(reinterpret_cast<unsigned long long *>(xo + c), (unsigned long long)q);
  }
}

// ---------------------------------------------------------------- attention + o projection
// One or two rows with a short context: attention and the o projection in one
// kernel.  The o projection is a sum over heads, o . W_o^T = sum_h o_h .
// W_o[:, h]^T, so workgroup (row block r, query head h, sequence b) computes
// head h's attention over the whole context (the g heads of a KV group read
// the same keys and values, which stay in L2), then multiplies o_h into the
// RB x hd block of W_o and adds the RB results into the residual.  The
// prologue is the split-KV kernel's (bias, RoPE, q rounded to f16; the new
// key and value come from LDS and one workgroup per KV head writes them into
// the cache); the four waves split the keys and meet in LDS.
template <int HD, int TPW>
__global__ void __launch_bounds__(256) dec_attn_o_kernel(DecAttnOArgs a) {
  constexpr int NW = 4, LPK = HD / 8, KPW = 64 / LPK, KSTEP = NW * KPW, HALF = HD / 2, U = 8;
  constexpr int RB = 64 * TPW;                 // W_o rows per workgroup
  static_assert(2 * HALF + HD <= 256, "one prologue element per thread");
  __shared__ float s_q[HD], s_k[HD], s_v[HD];
  __shared__ float s_m[NW], s_l[NW];
  __shared__ float s_o[NW][HD];
  __shared__ f16 s_oh[HD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slot = lane / LPK, dl = lane % LPK, d0 = dl * 8;
  const int i = lane & 15, g = lane >> 4;
  const int rb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int grp = a.n_heads / a.n_kv_heads, j = h / grp;
  const int pos = a.pos_dev[b];
  const int H = a.H;
  const int qd = a.n_heads * HD, kvd = a.n_kv_heads * HD, ncols = qd + 2 * kvd;
  const f16x8 zero = {};

  // prologue operands first (q of head h, new k and v of KV head j: their
  // projection sums, biases and the rotation at pos), so that bias + RoPE
  // runs while the W_o block and the cached keys are still arriving.
  // Thread e < HD handles a rotation pair (q for e < HALF, k above), thread
  // HD <= e < 2 HD one value of v; addresses are clamped, unused ones
  // discarded.
  const long long *acc = a.qkv_fix + (int64_t)b * ncols;
  const float2 *cs = a.rope + (int64_t)pos * HALF;
  const int pe = tid;
  const bool p_rot = pe < 2 * HALF, p_v = !p_rot && pe < 2 * HALF + HD;
  const int p_ii = (pe < HALF) ? pe : (p_rot ? pe - HALF : 0);
  const int p_c0 = p_rot ? ((pe < HALF) ? h * HD + p_ii : qd + j * HD + p_ii)
                         : qd + kvd + j * HD + (p_v ? pe - 2 * HALF : 0);
  const long long p_a0 = acc[p_c0], p_a1 = acc[p_rot ? p_c0 + HALF : p_c0];
  const float p_b0 = a.bias[p_c0], p_b1 = a.bias[p_rot ? p_c0 + HALF : p_c0];
  const float2 p_r = cs[p_ii];
  __builtin_amdgcn_sched_barrier(0);

  // W_o block: lane (i, g) holds row r0 + 16 tt + i, columns h hd + 32 s + 8 g
  const int r0 = rb * RB + wave * 16 * TPW;
  f16x8 wf[TPW][HD / 32];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int row = r0 + 16 * tt + i;
    // unit-tiled copy: row block min(row / 16, last), unit (h hd) / 32 + s
    const int rblk = min((r0 >> 4) + tt, (H - 1) >> 4);
#pragma unroll
    for (int s2 = 0; s2 < HD / 32; ++s2)
      wf[tt][s2] = a.w_o_tl ? load8((const f16 *)a.w_o_tl + ((int64_t)rblk * (qd >> 5) + ((h * HD) >> 5) + s2) * 512 + 8 * lane)
                            : load8((const f16 *)a.w_o + (int64_t)min(row, H - 1) * qd + h * HD + 32 * s2 + 8 * g);  // rows >= H: never stored
  }
  // cached keys 0 .. pos - 1: first batch before the prologue
  f16 *Kc = (f16 *)a.k_cache;
  f16 *Vc = (f16 *)a.v_cache;
  const int kc_end = pos;
  const int kstart = wave * KPW;
  f16x8 kr[U], vr[U];
  auto issue = [&](int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = kb + u * KSTEP + slot;
      // out-of-range keys get weight 0; their values must be finite
      const int tc = min(t, max(kc_end - 1, 0));
      const int64_t off = kv_offset(a.kv, a.n_kv_heads, HD, b, j, tc) + d0;
      const f16x8 kv = load8(Kc + off), vv = load8(Vc + off);
      kr[u] = t < kc_end ? kv : zero;
      vr[u] = t < kc_end ? vv : zero;
    }
  };
  issue(kstart);                   // unconditional: a wave with no keys loads clamped ones and zeroes them
  __builtin_amdgcn_sched_barrier(0);

  clear_share(a.clear, a.clear_n, (b * gridDim.y + h) * gridDim.x + rb, gridDim.x * gridDim.y * gridDim.z);

  const float qscale = a.softmax_scale * LOG2E;
  if (p_rot) {
    const float re = from_fix(p_a0) + p_b0, im = from_fix(p_a1) + p_b1;
    const float nre = re * p_r.x - im * p_r.y, nim = im * p_r.x + re * p_r.y;
    if (pe < HALF) {
      s_q[p_ii] = (float)(f16)nre * qscale;
      s_q[p_ii + HALF] = (float)(f16)nim * qscale;
    } else {
      s_k[p_ii] = (float)(f16)nre;
      s_k[p_ii + HALF] = (float)(f16)nim;
    }
  } else if (p_v) {
    s_v[pe - 2 * HALF] = (float)(f16)(from_fix(p_a0) + p_b0);
  }
  lds_barrier();                   // the W_o block and the keys stay in flight
  if (rb == 0 && h % grp == 0 && tid < HD) {
    const int64_t np = kv_offset(a.kv, a.n_kv_heads, HD, b, j, pos);
    Kc[np + tid] = (f16)s_k[tid];
    Vc[np + tid] = (f16)s_v[tid];
  }

  float q[8], o[8], m = -INFINITY, l = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    q[e] = s_q[d0 + e];
    o[e] = 0.f;
  }
  for (int kb = kstart; kb < kc_end; kb += U * KSTEP) {
    f16x8 kc[U], vc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kc[u] = kr[u];
      vc[u] = vr[u];
    }
    if (kb + U * KSTEP < kc_end) issue(kb + U * KSTEP);
    float sc[U];
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(q[e], (float)kc[u][e], d);
      d = group_sum<LPK>(d);
      sc[u] = (kb + u * KSTEP + slot < kc_end) ? d : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    const float corr = (m == -INFINITY) ? 0.f : exp2f(m - mx);
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= corr;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = (mx == -INFINITY) ? 0.f : exp2f(sc[u] - mx);
      lsum += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(p, (float)vc[u][e], o[e]);
    }
    l = l * corr + lsum;
    m = mx;
  }
  if (wave == 0 && slot == 0) {
    // the new key, from LDS
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) d = fmaf(q[e], s_k[d0 + e], d);
    d = group_sum<LPK>(d);
    const float mn = fmaxf(m, d);
    const float corr = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float p = exp2f(d - mn);
    l = l * corr + p;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(p, s_v[d0 + e], o[e] * corr);
    m = mn;
  }
  // merge the key slots of the wave, then the four waves
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float mo = __shfl_xor(m, off, 64);
    const float lo = __shfl_xor(l, off, 64);
    const float mn = fmaxf(m, mo);
    const float ca = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float cb = (mo == -INFINITY) ? 0.f : exp2f(mo - mn);
    l = l * ca + lo * cb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float oo = __shfl_xor(o[e], off, 64);
      o[e] = o[e] * ca + oo * cb;
    }
    m = mn;
  }
  if (slot == 0) {
    if (dl == 0) {
      s_m[wave] = m;
      s_l[wave] = l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_o[wave][d0 + e] = o[e];
  }
  __syncthreads();
  if (tid < HD) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = (s_m[w] == -INFINITY) ? 0.f : exp2f(s_m[w] - M);
      L = fmaf(c, s_l[w], L);
      O = fmaf(c, s_o[w][tid], O);
    }
    s_oh[tid] = (f16)(O / L);
  }
  __syncthreads();

  // o projection of this block: column 0 of the B operand is o_h
  f32x4 pacc[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) pacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < HD / 32; ++s2) {
    const f16x8 x = (i == 0) ? *reinterpret_cast<const f16x8 *>(&s_oh[32 * s2 + 8 * g]) : zero;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) pacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[tt][s2], x, pacc[tt], 0, 0, 0);
  }
  if (i == 0) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + 16 * tt + 4 * g + r;
        if (row < H) fix_add(a.x_out + (int64_t)b * H + row, pacc[tt][r] * a.o_scale, a.num_flag);
      }
  }
}

bool dec_attn_o_supported(int head_dim, int hidden) {
  return (head_dim == 64 || head_dim == 128) && hidden % 64 == 0;
}

hipError_t launch_dec_attn_o(hipStream_t s, const DecAttnOArgs &a) {
  if (!dec_attn_o_supported(a.head_dim, a.H) || a.batch < 1 || a.n_heads % a.n_kv_heads) return hipErrorInvalidValue;
  // 128-row blocks for the larger models: half the workgroups re-read the context
  const bool wide = a.H >= 1024;
  const int RB = wide ? 128 : 64;
  const dim3 grid((a.H + RB - 1) / RB, a.n_heads, a.batch);
  if (a.head_dim == 64) {
    if (wide) QW_LAUNCH((dec_attn_o_kernel<64, 2>), dim3(grid), dim3(256), 0, s, a);
    else QW_LAUNCH((dec_attn_o_kernel<64, 1>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (wide) QW_LAUNCH((dec_attn_o_kernel<128, 2>), dim3(grid), dim3(256), 0, s, a);
    else QW_LAUNCH((dec_attn_o_kernel<128, 1>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool dec_mlp_supported(int hidden, int inter) {
  return hidden % 128 == 0 && hidden <= 2048 && inter % MLP_F == 0;
}

// one row at H <= 1536 (the 1.5B model): late down-projection loads, two
// workgroups per CU (30.0 -> 28.7 us per launch, same box)
constexpr bool kMlpLateDown = true;

template <int NR>
hipError_t launch_dec_mlp32(hipStream_t s, const DecMlpArgs &a) {
  const dim3 grid(a.I / (2 * GU_BLOCK));
  if (a.H <= 1024)
    QW_LAUNCH((dec_mlp32_kernel<NR, 16, 8>), dim3(grid), dim3(512), 0, s, a);
  else if (a.H <= 1536 && kMlpLateDown && NR == 1)
    QW_LAUNCH((dec_mlp32_kernel<NR, 24, 16, true>), dim3(grid), dim3(512), 0, s, a);
  else if (a.H <= 1536)
    QW_LAUNCH((dec_mlp32_kernel<NR, 24, 16>), dim3(grid), dim3(512), 0, s, a);
  else
    QW_LAUNCH((dec_mlp32_kernel<NR, 32, 16>), dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

constexpr bool kMlp32 = true;

// One row at 1024 < H <= 1536: every weight requested at the start
// (dec_mlp16_kernel): 1.5B decode MLP 0.810 -> 0.645 ms per step (672 -> 752
// tokens/s).  At the 0.5B width the 32-feature kernel, which loads all its
// weights up front as well, stays faster (0.273 vs 0.291 ms per step).
constexpr bool kMlp16 = true;

hipError_t launch_dec_mlp(hipStream_t s, const DecMlpArgs &a) {
  if (!dec_mlp_supported(a.H, a.I) || a.M < 1 || a.M > 2) return hipErrorInvalidValue;
  // (up to H = 1536: at 2048 the 32 gate/up vectors per lane spill)
  if (kMlp16 && a.M == 1 && a.H % 128 == 0 && a.H > 1024 && a.H <= 1536 && a.I % GU_BLOCK == 0) {
    const size_t lds = (size_t)GU_BLOCK * a.H * 2;
    QW_LAUNCH((dec_mlp16_kernel<24>), dim3(a.I / GU_BLOCK), dim3(256), lds, s, a);
    return hipGetLastError();
  }
  if (kMlp32 && a.I % (2 * GU_BLOCK) == 0 && a.H >= 512)
    return a.M == 1 ? launch_dec_mlp32<1>(s, a) : launch_dec_mlp32<2>(s, a);
  const dim3 grid(a.I / MLP_F);
  const bool small = a.H <= 1024;
  if (a.M == 1) {
    if (small)
      QW_LAUNCH((dec_mlp_kernel<1, 8>), dim3(grid), dim3(256), 0, s, a);
    else
      QW_LAUNCH((dec_mlp_kernel<1, 16>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (small)
      QW_LAUNCH((dec_mlp_kernel<2, 8>), dim3(grid), dim3(256), 0, s, a);
    else
      QW_LAUNCH((dec_mlp_kernel<2, 16>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool decode_fast_supported(int head_dim, int group, int hidden, int q_dim, int inter) {
  return (head_dim == 32 || head_dim == 64 || head_dim == 128) && group >= 1 && group <= 8 && hidden % 32 == 0 &&
         q_dim % 32 == 0 && inter % GU_BLOCK == 0;
}

int dec_gemv_splits(int N, int K, int M, int target_groups) {
  const int nblk = (N + 63) / 64;
  const int units = K / 32;
  int splits = (target_groups + nblk - 1) / nblk;
  // at least 128 k per slice, 256 from K = 1024 on: every slice repeats the
  // norm prologue over the whole row (1.5B, one row: 1.553 -> 1.473 ms/step
  // with 256; 0.5B prefers 128: 0.6173 vs 0.6186 ms/step)
  const int minu = K >= 1024 ? 8 : 4;
  int max_splits = (units + minu - 1) / minu;
  // keep the atomic traffic (8 bytes per output per slice) under the weight bytes
  const int atomic_cap = (K * 2) / (8 * (M < 1 ? 1 : M));
  if (atomic_cap >= 1 && max_splits > atomic_cap) max_splits = atomic_cap;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return splits;
}

int dec_attn_splits(int batch, int n_kv_heads, int ctx, int target_groups) {
  int S = (target_groups + batch * n_kv_heads - 1) / (batch * n_kv_heads);
  const int by_len = (ctx + 63) / 64;          // at least 64 keys per split
  if (S > by_len) S = by_len;
  if (S > MERGE_MAX_S) S = MERGE_MAX_S;
  if (S < 1) S = 1;
  return S;
}

hipError_t launch_dec_embed(hipStream_t s, const int32_t *ids, int B, const void *emb, float emb_scale, int H, int V,
                            long long *x_fix, int *bad, long long *clr0, int64_t n0, long long *clr1, int64_t n1,
                            const RowNormOut &nout) {
  if (nout.w && nout.tiled && H % 32) return hipErrorInvalidValue;
  QW_LAUNCH((dec_embed_kernel), dim3(B), dim3(256), 0, s, ids, (const f16 *)emb, emb_scale, H, V, x_fix, bad, clr0, n0,
            clr1, n1, nout);
  return hipGetLastError();
}

int dec_norm_parts(int M, int N, int K) {
  if (M <= 2 || M > 32 || (K & 31)) return 0;          // the one/two-row kernels normalise their own operand
  const int rt = M <= 16 ? 1 : 2;                        // rows_plan's tile rows for FixAdd outputs
  const int parts = (N + 16 * rt - 1) / (16 * rt);
  if (parts > kNormPartsMax || parts > kSyncCounters) return 0;
  return parts;
}


hipError_t launch_dec_merge(hipStream_t s, const float *pm, const float *pl, const float *po, int S, int B, int nq,
                            int hd, void *o, bool tiled) {
  if (S < 1 || S > MERGE_MAX_S || hd > 128 || (tiled && (nq * hd) % 32)) return hipErrorInvalidValue;
  QW_LAUNCH((dec_merge_kernel), dim3(nq, B), dim3(128), 0, s, pm, pl, po, S, nq, hd, (f16 *)o, (int)tiled);
  return hipGetLastError();
}

hipError_t launch_dec_norm(hipStream_t s, const long long *x_fix, int64_t rep_stride, int B, int H,
                           const float *w, float eps, void *u) {
  QW_LAUNCH((dec_norm_kernel), dim3(B), dim3(256), 0, s, x_fix, rep_stride, H, w, eps, (f16 *)u);
  return hipGetLastError();
}

hipError_t launch_dec_end(hipStream_t s, const float *arg_v, const int *arg_i, int nblk, int B, int32_t *next,
                          int *pos_dev) {
  QW_LAUNCH((dec_end_kernel), dim3(B), dim3(256), 0, s, arg_v, arg_i, nblk, next, pos_dev);
  return hipGetLastError();
}

hipError_t launch_dec_gemv(hipStream_t s, const DecGemvArgs &in) {
  DecGemvArgs a = in;
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > 32 || (a.K & 31) || (a.lda & 7)) return hipErrorInvalidValue;
  if (a.act_mode == (int)DecAct::AttnMerge && (a.attn_splits < 1 || a.attn_splits > MERGE_MAX_S))
    return hipErrorInvalidValue;
  const bool rows_path = a.M > 2 && a.act_mode == (int)DecAct::F16 && !a.logits_mode;
  // the norm hand-off: u without 1/rms is read by the batched kernels and the
  // LM head on an f16 operand; it is produced by the batched residual projections
  if (a.nin.ss && (a.nin.parts < 1 || a.nin.parts > kNormPartsMax || a.act_mode != (int)DecAct::F16 ||
                   !(rows_path || a.logits_mode)))
    return hipErrorInvalidValue;
  if (a.nout.w && (!rows_path || a.swiglu_out || dec_norm_parts(a.M, a.N, a.K) == 0 || !a.nout.counters ||
                   !a.nout.u || !a.nout.ss || a.nout.ss_ld < dec_norm_parts(a.M, a.N, a.K) ||
                   (a.nout.tiled && a.N % 32)))
    return hipErrorInvalidValue;
  // tiled operands only in the batched kernels (tiled weights: every kernel)
  if ((a.act_tiled && !rows_path) || (a.act_tiled && a.swiglu_out && a.ldh % 32)) return hipErrorInvalidValue;
  const int units = a.K / 32;
  int splits = (a.logits_mode || a.swiglu_out) ? 1 : (a.splits < 1 ? 1 : a.splits);
  a.units_per_split = (units + splits - 1) / splits;
  splits = (units + a.units_per_split - 1) / a.units_per_split;
  // (the LM head stays on dec_gemv_kernel: 0.099 vs 0.110 ms per step at 8 rows)
  if (rows_path) {
    // batched rows: K split only for FixAdd outputs
    RowsPlan p = rows_plan(a, units);
    // the hand-off's column blocks are the tiles dec_norm_parts assumes
    if (a.nout.w && (a.N + 16 * p.rt - 1) / (16 * p.rt) != dec_norm_parts(a.M, a.N, a.K)) return hipErrorInvalidValue;
    a.units_per_split = (units + p.splits - 1) / p.splits;
    p.splits = (units + a.units_per_split - 1) / a.units_per_split;
    return a.M <= 16 ? launch_rows_nb<1>(s, a, p) : launch_rows_nb<2>(s, a, p);
  }
  dim3 grid((a.N + 63) / 64, splits);
  return a.M <= 16 ? launch_gemv_nb<1>(s, a, grid) : launch_gemv_nb<2>(s, a, grid);
}

hipError_t launch_dec_attention(hipStream_t s, const DecAttnArgs &a) {
  const int g = a.n_heads / a.n_kv_heads;
  if (a.o_tiled && (a.n_heads * a.head_dim) % 32) return hipErrorInvalidValue;
  dim3 grid(a.splits, a.n_kv_heads, a.batch);
  switch (a.head_dim) {
    case 32: return launch_attn_hd<32>(s, a, grid, g);
    case 64: return launch_attn_hd<64>(s, a, grid, g);
    case 128: return launch_attn_hd<128>(s, a, grid, g);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qw
