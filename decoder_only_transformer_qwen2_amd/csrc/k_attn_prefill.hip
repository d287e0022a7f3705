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
// workgroup is 4 waves x 32 queries of one head (two workgroups per CU).  The
// tiles go straight from memory into a ring of two LDS stages (the next key
// block in flight while one is multiplied), as swizzled 32-column sub-tiles
// (see swz).  V^T comes from a transposed copy of
// the prompt's V written once per layer (transpose_v_kernel), since
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

constexpr int BKEY = 64;  // keys per step (one cache block)
// Waves per workgroup and LDS stages (key blocks resident or in flight).
// Measured at 32 x 8192 (hd 128, ms per prefill): 4 waves x 2 stages 187.7
// (two workgroups per CU, whose barriers do not hold each other), 8 x 2
// 188.1, 8 x 4 193.3, 8 x 3 198.4; at 8 x 2048: 3.68, 3.88, 3.94, 4.01.
#ifndef QW_ATTN_WAVES
#define QW_ATTN_WAVES 4
#endif
#ifndef QW_ATTN_STAGES
#define QW_ATTN_STAGES 2
#endif
constexpr int AW = QW_ATTN_WAVES;
constexpr int AS = QW_ATTN_STAGES;
static_assert(AS >= 2 && AS <= 4, "stage ring");
constexpr int BQ = 32 * AW;   // queries per workgroup
constexpr float RESCALE_LOG2 = 8.0f;  // largest exponent (log2) a probability may reach before a rescale
constexpr int kTableLds = 512;        // paged cache: block ids held in LDS (contexts up to 32768 keys)

// 2^x with the hardware instruction alone: results below the smallest normal
// float flush to zero, which a probability can afford (it is rounded to f16)
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS tiles are kept as 32-column sub-tiles of 64-byte rows (four 16-byte
// chunks), chunk c of row r stored at c ^ swz(r): the 16 rows a fragment read
// touches then fall on distinct banks (the padded 272- and 144-byte rows of
// the first layout measured bank conflicts on 40% of the LDS cycles).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

// K rows are stored permuted: LDS row 32u + 16h + 4q + r holds key
// 32u + 8q + 4h + r (u, h < 2, q, r < 4), so that the S^T rows a lane owns
// (4q .. 4q+3 of tiles 2u and 2u+1) are 8 consecutive keys, which its V^T
// operand reads in one 16-byte load.
__device__ __forceinline__ int key_of_row(int row) {
  return (row & ~31) | (((row >> 2) & 3) << 3) | (((row >> 4) & 1) << 2) | (row & 3);
}

template <int HD>
__global__ void __launch_bounds__(64 * AW) __attribute__((amdgpu_waves_per_eu(2))) attn_prefill_kernel(AttnArgs a, int n_qt) {
  constexpr int KS = HD / 32;               // 32-wide d steps for S (K sub-tiles)
  constexpr int DT = HD / 16;               // 16-wide d tiles of O
  constexpr int KCH = KS * BKEY * 4;        // 16-byte chunks of a stage's K tile
  constexpr int VCH = 2 * HD * 4;           // of its V^T tile
  constexpr int NI = (KCH + VCH) / (64 * AW);   // loads per wave and stage
  static_assert((KCH + VCH) % (64 * AW) == 0 && KCH % 64 == 0, "whole load instructions per wave");
  __shared__ f16x8 sK[AS][KCH];   // [ks][key row][chunk]
  __shared__ f16x8 sV[AS][VCH];   // [u][d row][chunk]: keys 32u .. 32u + 31

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
    // wave-uniform values read from memory: said so, so that the block-table
    // lookups below are scalar loads (a vector load would need a vmcnt wait,
    // which would also wait for every key block in flight)
    const int it = __builtin_amdgcn_readfirstlane(a.tiles[w / nq]);
    b = it >> 16;
    qt = it & 0xffff;
    r0 = __builtin_amdgcn_readfirstlane(a.rag.cu[b]);
    P = __builtin_amdgcn_readfirstlane(a.rag.cu[b + 1]) - r0;
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

  // Key blocks go straight from memory into a ring of AS LDS stages: load
  // instruction n (n = NI * wave + q) of a stage fills its chunks 64n .. 64n
  // + 63, the K tile's first, then the V^T tile's; lane l's 16 bytes land at
  // chunk 64n + l, so each lane fetches the (row, chunk) that the swizzled,
  // permuted layout keeps there.  K rows past the prompt are clamped to its
  // last row (their scores are masked); V^T rows come from a transposed copy
  // of the prompt's V, zero past P in rows of round_up(P, 64) keys.
  const int q_last = min(P - 1, qt * BQ + BQ - 1);    // last query of the workgroup
  const int n_kb = q_last / BKEY + 1;                  // key blocks it needs
  const int PP = (P + BKEY - 1) / BKEY * BKEY;
  const int64_t vt_seq = a.tiles ? (int64_t)a.rag.pcu[b] : (int64_t)b * PP;   // padded rows before sequence b
  const f16 *Vt = (const f16 *)a.v_t + (vt_seq * a.n_kv_heads + (int64_t)j * PP) * HD;
  static_assert(BKEY == kKvBlock, "a key tile is one cache block");
  // A paged cache's block ids of this sequence go to LDS first: read in the
  // loop, the table (which the compiler cannot treat as read-only) would be a
  // vector load whose wait would also wait for every key block in flight.
  __shared__ int s_blk[kTableLds];
  const bool tbl_lds = a.kv.table != nullptr && n_kb <= kTableLds;
  if (tbl_lds) {
    for (int k = tid; k < n_kb; k += 64 * AW) s_blk[k] = a.kv.table[b * a.kv.blocks_per_seq + k];
    __syncthreads();
  }
  int src[NI], kkey[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int n = NI * wave + q, p = 64 * n + lane;
    if (n < KCH / 64) {
      const int ks = p / (4 * BKEY), row = (p >> 2) % BKEY, c = (p & 3) ^ swz(row);
      kkey[q] = key_of_row(row);
      src[q] = 32 * ks + 8 * c;
    } else {
      const int p2 = p - KCH, u = p2 / (4 * HD), row = (p2 >> 2) % HD, c = (p2 & 3) ^ swz(row);
      kkey[q] = 0;
      src[q] = row * PP + 32 * u + 8 * c;
    }
  }
  auto issue = [&](int kb) {
    const int st = kb % AS;
    int64_t koff;
    if (tbl_lds)
      koff = ((int64_t)s_blk[kb] * a.n_kv_heads + j) * (kKvBlock * HD);
    else
      koff = kv_offset(a.kv, a.n_kv_heads, HD, b, j, kb * BKEY);
    const f16 *Kt = Kc + koff;
    const int last_row = P - 1 - kb * BKEY;            // rows of the block past the prompt read this one
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int n = NI * wave + q;
      if (n < KCH / 64)
        dma16(Kt + (int64_t)min(kkey[q], last_row) * HD + src[q], &sK[st][64 * n]);
      else
        dma16(Vt + src[q] + kb * BKEY, &sV[st][64 * n - KCH]);
    }
  };

  // Online softmax state of the lane's query column (t): the reference m
  // (raw score units) that the exponents are taken from, and the running sum
  // l of the probabilities, which the matrix cores accumulate: a ones tile as
  // the A operand gives every row of lsum[t] the column sum of P^T, rescaled
  // with O.  The reference only moves when a score exceeds it by more than
  // RESCALE_LOG2 (in log2 units), so most blocks need no cross-lane maximum.
  const float sl2 = a.softmax_scale * 1.4426950408889634f;
  const float thr = RESCALE_LOG2 / sl2;              // the move threshold in raw score units
  float m[2] = {0.f, 0.f};
  f32x4 o[DT][2], lsum[2];
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int t = 0; t < 2; ++t) o[d][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  lsum[0] = lsum[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  f16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (f16)1.0f;

#pragma unroll
  for (int k = 0; k < AS - 1; ++k)
    if (k < n_kb) issue(k);
  // queries as B operands: lane (i, g) holds query q0 + 16t + i, dims 32s +
  // 8g .. +8.  Loaded after the first key blocks and awaited here with them:
  // the compiler's own wait for these loads would otherwise sit at their
  // first use inside the loop and, executed every iteration, wait for every
  // key block in flight.
  f16x8 qf[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int q = q0 + 16 * t + i;
      qf[t][s] = (q < P) ? *reinterpret_cast<const f16x8 *>(Q + (int64_t)q * qd + 32 * s + 8 * g) : zero8;
    }
  wait_vmcnt<0>();
  for (int kb = 0; kb < n_kb; ++kb) {
    const int cur = kb % AS;
    // this wave's share of stage kb is in (the later stages issued so far
    // may still be in flight); after the barrier every wave's is, and stage
    // kb - 1, whose buffer stage kb + AS - 1 reuses, has been consumed
    const int later = min(AS - 2, n_kb - 1 - kb);
    if (AS >= 4 && later == 2) wait_vmcnt<2 * NI * (AS >= 4)>();
    else if (AS >= 3 && later == 1) wait_vmcnt<NI * (AS >= 3)>();
    else wait_vmcnt<0>();
    stage_barrier();
    if (kb + AS - 1 < n_kb) issue(kb + AS - 1);
    const bool wave_active = kb * BKEY <= q0 + 31;     // any key of the block visible to this wave
    if (wave_active) {
      // S^T - m tiles: y = 16-key tile, t = 16-query tile; the accumulator
      // starts at -m, so the scores come out relative to the reference
      f32x4 s[4][2];
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int t = 0; t < 2; ++t) s[y][t] = f32x4{-m[t], -m[t], -m[t], -m[t]};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int row = 16 * y + i;
          const f16x8 kf = sK[cur][(ks * BKEY + row) * 4 + (g ^ swz(row))];
#pragma unroll
          for (int t = 0; t < 2; ++t) s[y][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[t][ks], s[y][t], 0, 0, 0);
        }
      // lane (i, g) holds, for S^T tile y, keys 32 (y / 2) + 8g + 4 (y % 2) + r
      // (the permuted K rows) of its query column.  Only blocks that reach
      // past the wave's first query are masked; masked scores are -inf, so
      // exp2 gives 0 without guards.
      const bool diag = kb * BKEY + BKEY - 1 > q0;
      float lm[2];
      if (diag) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int q = q0 + 16 * t + i;
          float mx = -INFINITY;
#pragma unroll
          for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = kb * BKEY + 32 * (y >> 1) + 8 * g + 4 * (y & 1) + r;
              const float v = (key <= q) ? s[y][t][r] : -INFINITY;
              s[y][t][r] = v;
              mx = fmaxf(mx, v);
            }
          lm[t] = mx;
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float mx = -INFINITY;
#pragma unroll
          for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[y][t][r]);
          lm[t] = mx;
        }
      }
      // Block 0 sets the reference (key 0 is visible to every query, so the
      // column maximum is finite); later blocks move it only for a column
      // with a score above m + thr.  Every lane of a column sees the same
      // column maximum, so the 4 lanes agree on the move.
      const bool first = kb == 0;
      if (__builtin_amdgcn_ballot_w64(first || lm[0] > thr || lm[1] > thr) != 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float cm = lm[t];
          cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
          cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
          const float delta = (first || cm > thr) ? cm : 0.f;
          if (delta != 0.f) {
            const float corr = first ? 0.f : exp2_raw(-delta * sl2);
#pragma unroll
            for (int d = 0; d < DT; ++d) o[d][t] *= corr;
            lsum[t] *= corr;
#pragma unroll
            for (int y = 0; y < 4; ++y)
#pragma unroll
              for (int r = 0; r < 4; ++r) s[y][t][r] -= delta;
            m[t] += delta;
          }
        }
      }
      // probabilities, packed as the B operand of step u: keys 32u + 8g + e
      // (tile 2u gives e < 4, tile 2u + 1 the rest)
      f16x8 pb[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb[t][u][e] = (f16)exp2_raw(s[2 * u][t][e] * sl2);
            pb[t][u][e + 4] = (f16)exp2_raw(s[2 * u + 1][t][e] * sl2);
          }
      // O^T += V^T . P^T (A operand from the transposed V tile with the same
      // key order) and l += ones . P^T
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const int row = 16 * d + i;
          const f16x8 vf = sV[cur][(u * HD + row) * 4 + (g ^ swz(row))];
#pragma unroll
          for (int t = 0; t < 2; ++t) o[d][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[t][u], o[d][t], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[t][u], lsum[t], 0, 0, 0);
      }
    }
  }

  // O^T: lane (i, g) holds dims 16d + 4g + r of query q0 + 16t + i
  f16 *O = (f16 *)a.o + (int64_t)r0 * qd + h * HD;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = q0 + 16 * t + i;
    if (q >= P) continue;
    const float inv = 1.0f / lsum[t][0];
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

int attn_prefill_query_tile() { return BQ; }

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
    case 32: QW_LAUNCH((attn_prefill_kernel<32>), dim3(grid), dim3(64 * AW), 0, s, a, n_qt); break;
    case 64: QW_LAUNCH((attn_prefill_kernel<64>), dim3(grid), dim3(64 * AW), 0, s, a, n_qt); break;
    case 128: QW_LAUNCH((attn_prefill_kernel<128>), dim3(grid), dim3(64 * AW), 0, s, a, n_qt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qw
