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
// tiles go straight from memory into LDS rings (global_load_lds) as swizzled
// 32-column sub-tiles (see swz).  V^T comes from a transposed copy of the
// prompt's V written once per layer (transpose_v_kernel), since transposing
// inside the kernel took 2-byte LDS stores with 16-way bank conflicts.  Work
// items are ordered heaviest (latest query tile) first and mapped so that the
// g query heads of a KV head and query tile run on the same XCD, where they
// share the K/V tiles in L2.
#include "qw_internal.h"

#include <math.h>

namespace qw {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BKEY = 64;  // keys per step (one cache block)
constexpr int BQ = 128;   // queries per workgroup: 4 waves x 32
constexpr float RESCALE_LOG2 = 8.0f;  // largest exponent (log2) a probability may reach before a rescale

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

// Software pipelined: block kb + 1's S^T = K . Q^T is issued in the same
// basic block as block kb's exponentials, so that a wave can keep the matrix
// cores busy while its softmax runs (the compiler interleaves them; a fixed
// interleave forced with sched_group_barrier measured slower).  K tiles take
// a ring of three LDS slots (block kb + 1 is resident while block kb is
// finished), V^T tiles a ring of two: 80 KB at hd 128, two workgroups per
// CU.  A paged cache's block ids of the first 128 blocks are held in two
// registers per lane (read with readlane), the rest read from the table.
template <int HD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) attn_prefill_kernel(AttnArgs a, int n_qt) {
  constexpr int PW = BQ / 32, PQ = BQ;      // waves, queries per workgroup
  constexpr int KS = HD / 32, DT = HD / 16;
  constexpr int KCH = KS * BKEY * 4, VCH = 2 * HD * 4;     // 16-byte chunks of a K / V^T tile
  constexpr int NK = KCH / 64 / PW, NV = VCH / 64 / PW;     // load instructions per wave and tile
  static_assert(KCH % (64 * PW) == 0 && VCH % (64 * PW) == 0, "whole load instructions per wave");
  __shared__ f16x8 sK[3][KCH];
  __shared__ f16x8 sV[2][VCH];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int nq = a.n_heads, grp = a.n_heads / a.n_kv_heads;
  const int total = a.tiles ? a.n_tiles * nq : n_qt * nq * (a.T / a.rows_per_seq);
  const int L = blockIdx.x;
  const int per_x = (total + 7) / 8;
  int w = (L % 8) * per_x + L / 8;
  if (w >= total) return;
  const int h = w % nq;
  int qt, b, P, r0;
  if (a.tiles) {
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
  const int q0 = qt * PQ + wave * 32;
  const int qd = nq * HD;
  const f16 *Q = (const f16 *)a.q + (int64_t)r0 * qd + h * HD;
  const f16 *Kc = (const f16 *)a.k_cache;
  const f16x8 zero8 = {};
  const int q_last = min(P - 1, qt * PQ + PQ - 1);
  const int n_kb = q_last / BKEY + 1;
  const int PP = (P + BKEY - 1) / BKEY * BKEY;
  const int64_t vt_seq = a.tiles ? (int64_t)a.rag.pcu[b] : (int64_t)b * PP;
  const f16 *Vt = (const f16 *)a.v_t + (vt_seq * a.n_kv_heads + (int64_t)j * PP) * HD;

  const bool paged = a.kv.table != nullptr;
  int blk_lo = 0, blk_hi = 0;
  if (paged) {
    const int *tb = a.kv.table + b * a.kv.blocks_per_seq;
    blk_lo = lane < n_kb ? tb[lane] : 0;
    blk_hi = 64 + lane < n_kb ? tb[64 + lane] : 0;
  }
  auto k_base = [&](int kb) -> int64_t {
    if (!paged) return kv_offset(a.kv, a.n_kv_heads, HD, b, j, kb * BKEY);
    const int blk = kb < 128 ? __builtin_amdgcn_readlane(kb < 64 ? blk_lo : blk_hi, kb & 63)
                             : a.kv.table[b * a.kv.blocks_per_seq + kb];
    return ((int64_t)blk * a.n_kv_heads + j) * (kKvBlock * HD);
  };
  int ksrc[NK], kkey[NK], vsrc[NV];
#pragma unroll
  for (int q = 0; q < NK; ++q) {
    const int p = 64 * (NK * wave + q) + lane;
    const int ks = p / (4 * BKEY), row = (p >> 2) % BKEY, c = (p & 3) ^ swz(row);
    kkey[q] = key_of_row(row);
    ksrc[q] = 32 * ks + 8 * c;
  }
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int p = 64 * (NV * wave + q) + lane;
    const int u = p / (4 * HD), row = (p >> 2) % HD, c = (p & 3) ^ swz(row);
    vsrc[q] = row * PP + 32 * u + 8 * c;
  }
  auto issue_k = [&](int kb) {
    const f16 *Kt = Kc + k_base(kb);
    const int last_row = P - 1 - kb * BKEY;
#pragma unroll
    for (int q = 0; q < NK; ++q)
      dma16(Kt + (int64_t)min(kkey[q], last_row) * HD + ksrc[q], &sK[kb % 3][64 * (NK * wave + q)]);
  };
  auto issue_v = [&](int kb) {
#pragma unroll
    for (int q = 0; q < NV; ++q) dma16(Vt + vsrc[q] + kb * BKEY, &sV[kb & 1][64 * (NV * wave + q)]);
  };

  const float sl2 = a.softmax_scale * 1.4426950408889634f;
  const float thr = RESCALE_LOG2 / sl2;
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

  issue_k(0);
  issue_v(0);
  if (n_kb > 1) issue_k(1);
  f16x8 qf[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const int q = q0 + 16 * t + i;
      qf[t][s2] = (q < P) ? *reinterpret_cast<const f16x8 *>(Q + (int64_t)q * qd + 32 * s2 + 8 * g) : zero8;
    }
  wait_vmcnt<0>();
  stage_barrier();

  // S^T of K tile in slot sl (accumulators start at zero: an inline constant
  // of the first MFMA, no register moves)
  auto smma = [&](f32x4 (&sc)[4][2], int sl) {
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int t = 0; t < 2; ++t) sc[y][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int row = 16 * y + i;
        const f16x8 kf = sK[sl][(ks * BKEY + row) * 4 + (g ^ swz(row))];
#pragma unroll
        for (int t = 0; t < 2; ++t) sc[y][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[t][ks], sc[y][t], 0, 0, 0);
      }
  };
  f32x4 sc[4][2];
  smma(sc, 0);

  // block kb: its scores in sc, block kb + 1's computed into sn; the loop
  // below alternates the two register sets (no copy between blocks)
  auto block = [&](int kb, f32x4 (&sc)[4][2], f32x4 (&sn)[4][2]) {
    if (kb > 0) {
      wait_vmcnt<0>();             // K of block kb + 1 and V^T of block kb (issued one step ago) are in
      stage_barrier();             // ... for every wave; block kb - 1 is finished by all
    }
    if (kb + 2 < n_kb) issue_k(kb + 2);
    if (kb + 1 < n_kb) issue_v(kb + 1);

    // masking, the column maxima and the rare reference move of block kb
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
            const float v = (key <= q) ? sc[y][t][r] : -INFINITY;
            sc[y][t][r] = v;
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
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[y][t][r]);
        lm[t] = mx;
      }
    }
    const bool first = kb == 0;
    if (__builtin_amdgcn_ballot_w64(first || lm[0] > m[0] + thr || lm[1] > m[1] + thr) != 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float cm = lm[t];
        cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
        cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
        if (first || cm > m[t] + thr) {
          const float corr = first ? 0.f : exp2_raw((m[t] - cm) * sl2);
#pragma unroll
          for (int d = 0; d < DT; ++d) o[d][t] *= corr;
          lsum[t] *= corr;
          m[t] = cm;
        }
      }
    }
    // p = 2^((s - m) sl2), the reference folded into one fused multiply-add
    const float msl[2] = {-m[0] * sl2, -m[1] * sl2};

    // one basic block: S^T of block kb + 1 (after the last iteration a
    // stale slot, never used), the probabilities of block kb, P.V
    smma(sn, (kb + 1) % 3);
    f16x8 pb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[t][u][e] = (f16)exp2_raw(fmaf(sc[2 * u][t][e], sl2, msl[t]));
          pb[t][u][e + 4] = (f16)exp2_raw(fmaf(sc[2 * u + 1][t][e], sl2, msl[t]));
        }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        const int row = 16 * d + i;
        const f16x8 vf = sV[kb & 1][(u * HD + row) * 4 + (g ^ swz(row))];
#pragma unroll
        for (int t = 0; t < 2; ++t) o[d][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[t][u], o[d][t], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[t][u], lsum[t], 0, 0, 0);
    }
  };
  f32x4 sn[4][2];
  for (int kb = 0; kb < n_kb; kb += 2) {
    block(kb, sc, sn);
    if (kb + 1 < n_kb) block(kb + 1, sn, sc);
  }

  // o rows, row-major or unit-tiled (the o projection's operand): a lane's 4
  // dims are consecutive within one 8-dim chunk either way
  f16 *O = (f16 *)a.o;
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
      const int row = r0 + q, col = h * HD + 16 * d + 4 * g;
      *reinterpret_cast<f16x4 *>(O + (a.o_tiled ? tile_off(row, col, qd) : (int64_t)row * qd + col)) = v;
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
    case 32: QW_LAUNCH((attn_prefill_kernel<32>), dim3(grid), dim3(256), 0, s, a, n_qt); break;
    case 64: QW_LAUNCH((attn_prefill_kernel<64>), dim3(grid), dim3(256), 0, s, a, n_qt); break;
    case 128: QW_LAUNCH((attn_prefill_kernel<128>), dim3(grid), dim3(256), 0, s, a, n_qt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qw
