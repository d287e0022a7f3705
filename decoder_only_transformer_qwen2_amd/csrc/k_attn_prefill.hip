// Prefill attention on the matrix cores: causal grouped-query attention of
// every prompt row against the keys/values already in the cache ("LLM
// Speedrun: Architecture", sections "Attention", "Every token with every
// other token, even the future ones?" and "Grouped Query Attention GQA";
// query head h reads KV head floor(h / g)).
//
// Flash-style: keys are visited 64 at a time with an online softmax, so the
// score matrix is never stored.  The products are taken transposed,
//   S^T = K . Q^T          (A = K tile rows, B = query rows)
//   O^T += V^T . P^T       (A = V^T from LDS, B = probabilities)
// which leaves each lane owning ONE query column of S^T and O^T: the running
// max / sum / rescale of the online softmax are per-lane scalars, and the
// probabilities already sit in the B-operand layout of the second product, so
// P never goes through LDS.  The K rows of each 32-key step are stored in a
// permuted order so that the 8 probabilities a lane holds for a step are 8
// consecutive keys, which its V^T operand reads in one 16-byte load.  A
// workgroup is 4 waves x 32 queries of
// one head; the K tile ([key][d]) and the V^T tile ([d][key]) are staged in
// LDS with two buffers, both as 16-byte vectors: V^T comes from a transposed
// copy of the prompt's V written once per layer (transpose_v_kernel), since
// transposing inside the kernel took 2-byte LDS stores with 16-way bank
// conflicts.  Work items are ordered heaviest (latest
// query tile) first and mapped so that the g query heads of a KV head and
// query tile run on the same XCD, where they share the K/V tiles in L2.
#include "qw_internal.h"

#include <math.h>

namespace qw {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BQ = 128;   // queries per workgroup (4 waves x 32)
constexpr int BKEY = 64;  // keys per step
constexpr float RESCALE_LOG2 = 8.0f;  // largest exponent (log2) a probability may reach before a rescale

// 2^x with the hardware instruction alone: results below the smallest normal
// float flush to zero, which a probability can afford (it is rounded to f16)
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int HD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) attn_prefill_kernel(AttnArgs a, int n_qt) {
  constexpr int KP = HD + 8;          // padded K row
  constexpr int VP = BKEY + 8;        // padded V^T row
  constexpr int KS = HD / 32;         // 32-wide d steps for S
  constexpr int DT = HD / 16;         // 16-wide d tiles of O
  constexpr int VEC = BKEY * HD / 8;  // 16-byte vectors per K (or V) tile
  constexpr int VPT = VEC / 256;      // per thread
  __shared__ f16 sK[2][BKEY][KP];
  __shared__ f16 sV[2][HD][VP];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int nq = a.n_heads, grp = a.n_heads / a.n_kv_heads;
  // work item: heaviest query tiles first; the g heads of a group adjacent,
  // and adjacent items on one XCD (workgroups go round-robin over 8 XCDs).
  // Ragged batches take (sequence, query tile) from a list the host ordered
  // so that each XCD's range starts heaviest and the ranges weigh the same.
  const int total = a.tiles ? a.n_tiles * nq : n_qt * nq * (a.T / a.rows_per_seq);
  const int L = blockIdx.x;
  const int per_x = (total + 7) / 8;
  int w = (L % 8) * per_x + L / 8;
  if (w >= total) return;
  const int h = w % nq;
  int qt, b, P, r0;
  if (a.tiles) {
    const int it = a.tiles[w / nq];
    b = it >> 16;
    qt = it & 0xffff;
    r0 = a.rag.cu[b];
    P = a.rag.cu[b + 1] - r0;
  } else {
    P = a.rows_per_seq;
    qt = n_qt - 1 - (w / nq) % n_qt;
    b = w / (nq * n_qt);
    r0 = b * P;
  }
  const int j = h / grp;
  const int q0 = qt * BQ + wave * 32;                 // this wave's first query
  const int qd = nq * HD;

  const f16 *Q = (const f16 *)a.q + (int64_t)r0 * qd + h * HD;
  const f16 *Kc = (const f16 *)a.k_cache;
  const f16x8 zero8 = {};

  // queries as B operands: lane (i, g) holds query q0 + 16t + i, dims 32s + 8g .. +8
  f16x8 qf[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int q = q0 + 16 * t + i;
      qf[t][s] = (q < P) ? *reinterpret_cast<const f16x8 *>(Q + (int64_t)q * qd + 32 * s + 8 * g) : zero8;
    }

  const float sl2 = a.softmax_scale * 1.4426950408889634f;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4 o[DT][2];
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int t = 0; t < 2; ++t) o[d][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int q_last = min(P - 1, qt * BQ + BQ - 1);    // last query of the workgroup
  const int n_kb = q_last / BKEY + 1;                  // key blocks it needs
  f16x8 rk[VPT], rv[VPT];
  // K rows [key][d] from the cache, V^T rows [d][key] from the transposed
  // copy (rows of round_up(P, 64) keys, zero past P): both as 16-byte vectors
  const int PP = (P + BKEY - 1) / BKEY * BKEY;
  const int64_t vt_seq = a.tiles ? (int64_t)a.rag.pcu[b] : (int64_t)b * PP;   // padded rows before sequence b
  const f16 *Vt = (const f16 *)a.v_t + (vt_seq * a.n_kv_heads + (int64_t)j * PP) * HD;
  static_assert(BKEY == kKvBlock, "a key tile is one cache block");
  auto gload = [&](int kb) {
    const f16 *Kt = Kc + kv_offset(a.kv, a.n_kv_heads, HD, b, j, kb * BKEY);
#pragma unroll
    for (int t = 0; t < VPT; ++t) {
      const int v = tid + 256 * t;
      const int kk = v / (HD / 8), key = kb * BKEY + kk, c = (v % (HD / 8)) * 8;
      rk[t] = key < P ? *reinterpret_cast<const f16x8 *>(Kt + (int64_t)kk * HD + c) : zero8;
      const int d = v / (BKEY / 8), kc = (v % (BKEY / 8)) * 8;
      rv[t] = *reinterpret_cast<const f16x8 *>(Vt + (int64_t)d * PP + kb * BKEY + kc);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int t = 0; t < VPT; ++t) {
      const int v = tid + 256 * t;
      const int key = v / (HD / 8), c = (v % (HD / 8)) * 8;
      // LDS row 32u + 16h + 4q + r holds key 32u + 8q + 4h + r (u, h < 2, q,
      // r < 4): the S^T rows a lane owns (4q .. 4q+3 of tiles 2u and 2u+1)
      // are then 8 consecutive keys, read from V^T in one 16-byte load
      const int krow = (key & ~31) | (((key >> 2) & 1) << 4) | (((key >> 3) & 3) << 2) | (key & 3);
      *reinterpret_cast<f16x8 *>(&sK[buf][krow][c]) = rk[t];
      const int d = v / (BKEY / 8), kc = (v % (BKEY / 8)) * 8;
      *reinterpret_cast<f16x8 *>(&sV[buf][d][kc]) = rv[t];
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < n_kb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < n_kb) gload(kb + 1);
    const bool wave_active = kb * BKEY <= q0 + 31;     // any key of the block visible to this wave
    if (wave_active) {
      // S^T tiles: y = 16-key tile, t = 16-query tile
      f32x4 s[4][2];
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int t = 0; t < 2; ++t) s[y][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const f16x8 kf = *reinterpret_cast<const f16x8 *>(&sK[cur][16 * y + i][32 * ks + 8 * g]);
#pragma unroll
          for (int t = 0; t < 2; ++t) s[y][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[t][ks], s[y][t], 0, 0, 0);
        }
      // online softmax per query column; lane (i, g) holds, for S^T tile y,
      // keys 32 (y / 2) + 8g + 4 (y % 2) + r (the permuted K rows).
      // Scores stay unscaled: the scale goes into the exponent's FMA, and
      // only blocks that reach past the wave's first query are masked.  The
      // running max is finite from block 0 on (key 0 is visible to every
      // query), and masked scores are -inf, so exp2 needs no guards.
      const bool diag = kb * BKEY + BKEY - 1 > q0;
      f16x8 pb[2][2];
      float corr[2];
      bool any_move = false;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int q = q0 + 16 * t + i;
        float mx = -INFINITY;
        if (diag) {
#pragma unroll
          for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = kb * BKEY + 32 * (y >> 1) + 8 * g + 4 * (y & 1) + r;
              const float v = (key <= q) ? s[y][t][r] : -INFINITY;
              s[y][t][r] = v;
              mx = fmaxf(mx, v);
            }
        } else {
#pragma unroll
          for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[y][t][r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // The reference point of the exponent only moves when the block's
        // max exceeds it by more than RESCALE_LOG2 (in log2 units): softmax
        // is invariant to the reference, and a stale one keeps every p below
        // 2^RESCALE_LOG2.  Block 0 always moves it off -inf.
        const float mn = fmaxf(m[t], mx);
        const bool move = (mn - m[t]) * sl2 > RESCALE_LOG2;
        const float mref = move ? mn : m[t];
        corr[t] = move ? exp2_raw((m[t] - mn) * sl2) : 1.0f;
        any_move |= move;
        const float nb = -mref * sl2;
        float sum = 0.f;
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = exp2_raw(fmaf(s[y][t][r], sl2, nb));
            s[y][t][r] = p;
            sum += p;
          }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        l[t] = l[t] * corr[t] + sum;
        m[t] = mref;
        // B operand of step u: keys 32u + 8g + e (tile 2u gives e < 4, tile 2u + 1 the rest)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb[t][u][e] = (f16)s[2 * u][t][e];
            pb[t][u][e + 4] = (f16)s[2 * u + 1][t][e];
          }
      }
      // rescale the accumulators only when some query of the wave moved its reference
      if (__builtin_amdgcn_ballot_w64(any_move) != 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int d = 0; d < DT; ++d) o[d][t] *= corr[t];
      }
      // O^T += V^T . P^T, A operand from the transposed V tile with the same key order
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const f16x8 vf = *reinterpret_cast<const f16x8 *>(&sV[cur][16 * d + i][32 * u + 8 * g]);
#pragma unroll
          for (int t = 0; t < 2; ++t) o[d][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[t][u], o[d][t], 0, 0, 0);
        }
    }
    if (kb + 1 < n_kb) lstore(cur ^ 1);
    __syncthreads();
  }

  // O^T: lane (i, g) holds dims 16d + 4g + r of query q0 + 16t + i
  f16 *O = (f16 *)a.o + (int64_t)r0 * qd + h * HD;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = q0 + 16 * t + i;
    if (q >= P) continue;
    const float inv = 1.0f / l[t];
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      f16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (f16)(o[d][t][r] * inv);
      *reinterpret_cast<f16x4 *>(O + (int64_t)q * qd + 16 * d + 4 * g) = v;
    }
  }
}

}  // namespace

bool attn_prefill_supported(int head_dim) { return head_dim == 32 || head_dim == 64 || head_dim == 128; }

// 64 keys x 64 dims per workgroup through LDS, so that both the reads (rows
// of the cache) and the writes (rows of V^T) are contiguous.  Sequence b is
// P keys long (ragged: cu[b+1] - cu[b]); its V^T rows are round_up(P, 64)
// long and start at (padded rows before b) * nkv * hd.
__global__ void __launch_bounds__(256) transpose_v_kernel(const f16 *v_cache, KvMap kv, RaggedRows rag, int n_kv_heads,
                                                          int hd, int P_eq, f16 *v_t) {
  __shared__ f16 tile[64][66];
  const int t0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const int b = blockIdx.z / n_kv_heads, j = blockIdx.z % n_kv_heads;
  const int P = rag.cu ? rag.cu[b + 1] - rag.cu[b] : P_eq;
  const int PP = (P + 63) / 64 * 64;
  if (t0 >= PP) return;                         // past this sequence (ragged: shorter than the longest)
  const int64_t seq_rows = rag.cu ? (int64_t)rag.pcu[b] : (int64_t)b * PP;
  const f16 *src = v_cache + kv_offset(kv, n_kv_heads, hd, b, j, t0);   // keys t0 .. t0 + 63: one cache block
  f16 *dst = v_t + (seq_rows * n_kv_heads + (int64_t)j * PP) * hd;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e / 64, c = e % 64;            // key t0 + r, dim d0 + c
    const int key = t0 + r, d = d0 + c;
    tile[r][c] = (key < P && d < hd) ? src[(int64_t)r * hd + d] : (f16)0.f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e / 64, c = e % 64;            // dim r, key c
    const int d = d0 + r, key = t0 + c;
    if (d < hd && key < PP) dst[(int64_t)d * PP + key] = tile[c][r];
  }
}

hipError_t launch_transpose_v(hipStream_t s, const void *v_cache, const KvMap &kv, const RaggedRows &rag, int B,
                              int n_kv_heads, int head_dim, int P, int max_len, void *v_t) {
  if (max_len <= 0) return hipSuccess;
  const int PP = (max_len + BKEY - 1) / BKEY * BKEY;
  dim3 grid(PP / 64, (head_dim + 63) / 64, B * n_kv_heads);
  QW_LAUNCH((transpose_v_kernel), dim3(grid), dim3(256), 0, s, (const f16 *)v_cache, kv, rag, n_kv_heads, head_dim,
            P, (f16 *)v_t);
  return hipGetLastError();
}

hipError_t launch_attention_prefill(hipStream_t s, const AttnArgs &a) {
  if (a.T <= 0) return hipSuccess;
  if (a.pos0_dev || a.pos0 != 0) return hipErrorInvalidValue;
  int n_qt = 0, total;
  if (a.tiles) {
    if (!a.rag.cu || a.n_tiles < 1) return hipErrorInvalidValue;
    total = a.n_tiles * a.n_heads;
  } else {
    if (a.T % a.rows_per_seq) return hipErrorInvalidValue;
    n_qt = (a.rows_per_seq + BQ - 1) / BQ;
    total = n_qt * a.n_heads * (a.T / a.rows_per_seq);
  }
  const int per_x = (total + 7) / 8;
  dim3 grid(per_x * 8);
  switch (a.head_dim) {
    case 32: QW_LAUNCH((attn_prefill_kernel<32>), dim3(grid), dim3(256), 0, s, a, n_qt); break;
    case 64: QW_LAUNCH((attn_prefill_kernel<64>), dim3(grid), dim3(256), 0, s, a, n_qt); break;
    case 128: QW_LAUNCH((attn_prefill_kernel<128>), dim3(grid), dim3(256), 0, s, a, n_qt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qw
