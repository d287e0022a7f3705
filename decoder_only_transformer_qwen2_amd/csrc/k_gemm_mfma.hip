// Prefill projections on the matrix cores: C[M, N] = A[M, K] . W[N, K]^T with
// f16 operands and fp32 accumulation (v_mfma_f32_16x16x32_f16), for the
// q/k/v, o, gate/up and down projections and the LM head over all prompt
// rows at once ("Building a Qwen2.5-1.5B Inference Engine From Scratch",
// section 1: prefill processes every prompt token in parallel, which makes it
// compute-bound).  Epilogues as in the generic kernel: store fp32, add into
// the fp32 residual stream, or silu(gate) * up over the GU_BLOCK-interleaved
// gate/up rows.
//
// Few output tiles (short prompts) leave most of the chip idle, so K can be
// split over gridDim.z: each slice stores its raw fp32 tile in a workspace and
// a second kernel adds the slices in slice order (deterministic) and applies
// the epilogue.
//
// Two kernels share the epilogues:
//  * gemm_lds_kernel (K % 32 == 0, the model's shapes): operands go straight
//    from memory into LDS (16 bytes per lane) through a ring of BK = 32
//    stages, with no staging registers; 256 x 256 tiles on 8 waves when there
//    are enough of them (half the operand bytes per FLOP of 128 x 128:
//    the 128 x 128 version is bound by operand traffic from L2, not by MFMA),
//    128 x 128 on 4 waves otherwise.
//  * gemm_mfma_kernel (any K % 8 == 0): 128 x 128 x 64 tiles, both operands
//    staged through registers into two LDS buffers (rows padded by 16 bytes).
// Both order their tiles per XCD (see the kernels).
#include "qw_internal.h"

namespace qw {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDP = BK + 8;           // padded LDS row (f16 elements)

template <Epi EPI>
__global__ void __launch_bounds__(256) gemm_mfma_kernel(GemmArgs a) {
  __shared__ f16 sA[2][BM][LDP];
  __shared__ f16 sB[2][BN][LDP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;          // wave's 64 x 64 sub-tile
  // Tile order: workgroups are dealt round-robin to the 8 XCDs, each with its
  // own L2.  Workgroup L therefore takes tile t = (L % 8) * per_x + L / 8, so
  // each XCD works through a contiguous range of t; t runs over groups of
  // GM row tiles, column by column, so the tiles in flight on one XCD share
  // their A rows and B columns in that XCD's L2.
  constexpr int GM = 4;
  const int TM = (a.M + BM - 1) / BM, TN = (a.N + BN - 1) / BN;
  const int per_x = (TM * TN + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per_x + (int)(blockIdx.x / 8);
  if (t >= TM * TN) return;
  const int grp = t / (GM * TN), within = t % (GM * TN);
  const int gsz = min(GM, TM - grp * GM);
  const int m0 = (grp * GM + within % gsz) * BM, n0 = (within / gsz) * BN;
  const f16 *A = (const f16 *)a.A;
  const f16 *W = (const f16 *)a.W;
  const f16x8 zero = {};

  // global -> register staging: 1024 16-byte vectors per operand tile, 4 per thread
  f16x8 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int v = tid + 256 * t;
      const int r = v >> 3, c = (v & 7) * 8;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + c;
      ra[t] = (gm < a.M && gk < a.K) ? *reinterpret_cast<const f16x8 *>(A + (int64_t)gm * a.lda + gk) : zero;
      rb[t] = (gn < a.N && gk < a.K) ? *reinterpret_cast<const f16x8 *>(W + (int64_t)gn * a.K + gk) : zero;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int v = tid + 256 * t;
      const int r = v >> 3, c = (v & 7) * 8;
      *reinterpret_cast<f16x8 *>(&sA[buf][r][c]) = ra[t];
      *reinterpret_cast<f16x8 *>(&sB[buf][r][c]) = rb[t];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K range of this slice (whole BK tiles)
  const int KT_all = (a.K + BK - 1) / BK;
  const int kt_per = (KT_all + gridDim.z - 1) / gridDim.z;
  const int kt0 = blockIdx.z * kt_per;
  const int KT = max(0, min(KT_all, kt0 + kt_per) - kt0);
  const int kbase = kt0 * BK;
  gload(kbase);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kbase + (kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      f16x8 fa[4], fb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        fa[x] = *reinterpret_cast<const f16x8 *>(&sA[cur][wm * 64 + x * 16 + i][ks + 8 * g]);
#pragma unroll
      for (int y = 0; y < 4; ++y)
        fb[y] = *reinterpret_cast<const f16x8 *>(&sB[cur][wn * 64 + y * 16 + i][ks + 8 * g]);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

  // acc[x][y]: lane (i, g) holds rows 4g..4g+3 of column i of MFMA tile (x, y)
  if (gridDim.z > 1) {
    float *ws = a.ws + (int64_t)blockIdx.z * a.M * a.N;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int col = n0 + wn * 64 + y * 16 + i;
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 64 + x * 16 + 4 * g + r;
          if (row < a.M) ws[(int64_t)row * a.N + col] = acc[x][y][r];
        }
      }
    return;
  }
  if constexpr (EPI == Epi::SwiGLU) {
    // the wave's 64 columns are two (gate block, up block) pairs: y = 0/1 and 2/3
    f16 *out = (f16 *)a.act_out;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int f = (n0 + wn * 64) / 2 + p * GU_BLOCK + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 64 + x * 16 + 4 * g + r;
          if (row < a.M && f < a.N / 2) {
            const float gt = acc[x][2 * p][r] * a.scale, up = acc[x][2 * p + 1][r] * a.scale;
            out[a.h_tiled ? tile_off(row, f, a.ldo) : (int64_t)row * a.ldo + f] = (f16)(silu_f(gt) * up);
          }
        }
      }
  } else {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int col = n0 + wn * 64 + y * 16 + i;
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 64 + x * 16 + 4 * g + r;
          if (row >= a.M) continue;
          float *o = a.out_f32 + (int64_t)row * a.ldo + col;
          const float v = acc[x][y][r] * a.scale;
          if constexpr (EPI == Epi::ResidAdd)
            *o += v;
          else
            *o = v;
        }
      }
  }
}

// The same tile with the operands loaded straight into LDS
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS base
// + 16 * lane) through a ring of four BK = 32 stages, three of them in flight
// while one is multiplied, and no staging registers.  A stage holds 128 rows x
// 4 chunks of 16 bytes per operand, chunk c of row r stored at position
// c ^ ((r >> 1) & 3), so the 16 rows an MFMA operand read touches spread over
// the banks.  Rows past M or N load a clamped row and are never stored;
// K % 32 == 0.
constexpr int LK = 32, NSTG = 4;
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 3; }

// The 256 x 256 kernel's residual-add and SwiGLU epilogues through LDS
#ifndef QW_ROW_EPILOGUE
#define QW_ROW_EPILOGUE 1
#endif
constexpr bool kRowEpilogue = QW_ROW_EPILOGUE;

// Epi::QkvRope.  Sequence and position of prompt row `row` (equal-length
// sequences of rows_per_seq rows, or the ragged ones of rag).
__device__ __forceinline__ void qkv_row_pos(const QkvRopeArgs &q, int row, int &b, int &pos) {
  if (q.rag.cu) {
    b = ragged_seq(q.rag.cu, q.rag.n, row);
    pos = row - q.rag.cu[b];
  } else {
    b = row / q.rows_per_seq;
    pos = row - b * q.rows_per_seq;
  }
}
// Row `row` (sequence b, position pos): the projections of columns oc_lo
// and oc_hi (for q and k, a rotation pair d and d + hd/2; for v
// two columns of one head) plus their biases; q and k rotated by the
// split-half RoPE at pos ("LLM Speedrun: Architecture", "Split-half RoPE
// implementation"), then q to q_out and k, v into the cache, rounded to f16
// once -- the arithmetic of the separate bias + RoPE + cache-write kernel.
__device__ __forceinline__ void qkv_rope_store(const QkvRopeArgs &q, int row, int b, int pos, int oc_lo, int oc_hi,
                                               float vlo, float vhi) {
  const int hd = q.head_dim, half = hd >> 1, qd = q.n_heads * hd, kvd = q.n_kv_heads * hd;
  const float re = vlo + q.bias[oc_lo], im = vhi + q.bias[oc_hi];
  if (oc_lo < qd + kvd) {
    const int d = oc_lo % hd;
    const float2 cs = q.rope[(int64_t)pos * half + d];
    const float nre = re * cs.x - im * cs.y;
    const float nim = im * cs.x + re * cs.y;
    f16 *o;
    if (oc_lo < qd)
      o = (f16 *)q.q_out + (int64_t)row * qd + oc_lo;
    else
      o = (f16 *)q.k_cache + kv_offset(q.kv, q.n_kv_heads, hd, b, (oc_lo - qd) / hd, pos) + d;
    o[0] = (f16)nre;
    o[half] = (f16)nim;
  } else {
    const int c = oc_lo - qd - kvd;
    f16 *o = (f16 *)q.v_cache + kv_offset(q.kv, q.n_kv_heads, hd, b, c / hd, pos);
    o[c % hd] = (f16)re;
    o[(oc_hi - qd - kvd) % hd] = (f16)im;
  }
}

// TL: A and W unit-tiled (qw_internal.h; a.W is then the tiled weight copy):
// a DMA instruction reads one 1 KB tile (16 rows x 32 k) and lands it in the
// same order, which is also the MFMA operand order, so fragments are read
// back as 1 KB contiguous per wave (no swizzle needed).  Row-major operands
// take 16 pieces of 64 B per instruction, 2.5x the cost of contiguous reads
// even from L2 (measured).
template <Epi EPI, int TBM, int TBN, int WVM, int WVN, int NS, bool FP = false, bool TL = false>
__global__ void __launch_bounds__(64 * WVM * WVN) gemm_lds_kernel(GemmArgs a) {
  constexpr int NWV = WVM * WVN;                  // waves
  constexpr int XT = TBM / WVM / 16, YT = TBN / WVN / 16;   // MFMA tiles per wave
  constexpr int QA = TBM / 16 / NWV, QB = TBN / 16 / NWV;   // load instructions per wave and stage
  static_assert((TBN / WVN) % (2 * GU_BLOCK) == 0, "a wave's columns hold whole gate/up pairs");
  // one LDS block: the operand stages, and after the K loop the staging of
  // the output tile for a row-contiguous epilogue
  __shared__ f16x8 s_lds[NS * (TBM + TBN) * 4];
  f16x8 (*sA)[TBM * 4] = reinterpret_cast<f16x8 (*)[TBM * 4]>(s_lds);
  f16x8 (*sB)[TBN * 4] = reinterpret_cast<f16x8 (*)[TBN * 4]>(s_lds + NS * TBM * 4);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int wm = wave / WVN, wn = wave % WVN;
  constexpr int GM = 4;
  const int TM = (a.M + TBM - 1) / TBM, TN = (a.N + TBN - 1) / TBN;
  const int per_x = (TM * TN + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per_x + (int)(blockIdx.x / 8);
  if (t >= TM * TN) return;
  const int grp = t / (GM * TN), within = t % (GM * TN);
  const int gsz = min(GM, TM - grp * GM);
  const int m0 = (grp * GM + within % gsz) * TBM, n0 = (within / gsz) * TBN;
  const f16 *A = (const f16 *)a.A;
  const f16 *W = (const f16 *)a.W;

  // wave w, instruction q covers stage positions 64 (QA w + q) .. + 63, i.e.
  // rows 16 (QA w + q) + lane / 4 (likewise for B)
  const int KT_all = a.K / LK;
  const int kt_per = (KT_all + gridDim.z - 1) / gridDim.z;
  const int kt0 = blockIdx.z * kt_per;
  const int KT = max(0, min(KT_all, kt0 + kt_per) - kt0);
  const f16 *srcA[QA], *srcB[QB];
  if constexpr (TL) {
    // row block (clamped to the last one; rows past M or N are never stored)
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int rb = min(m0 / 16 + QA * wave + q, (a.M - 1) / 16);
      srcA[q] = A + ((int64_t)rb * (a.K / LK) + kt0) * 512 + 8 * lane;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int rb = min(n0 / 16 + QB * wave + q, (a.N - 1) / 16);
      srcB[q] = W + ((int64_t)rb * (a.K / LK) + kt0) * 512 + 8 * lane;
    }
  } else {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int row = 16 * (QA * wave + q) + (lane >> 2);
      const int c = (lane & 3) ^ lds_swz(row);
      srcA[q] = A + (int64_t)min(m0 + row, a.M - 1) * a.lda + (int64_t)kt0 * LK + 8 * c;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int row = 16 * (QB * wave + q) + (lane >> 2);
      const int c = (lane & 3) ^ lds_swz(row);
      srcB[q] = W + (int64_t)min(n0 + row, a.N - 1) * a.K + (int64_t)kt0 * LK + 8 * c;
    }
  }
  constexpr int KSTEP = TL ? 512 : LK;            // elements between consecutive K stages of a source
  auto issue = [&](int kt) {
    const int st = kt % NS;
#pragma unroll
    for (int q = 0; q < QA; ++q) dma16(srcA[q] + kt * KSTEP, &sA[st][64 * (QA * wave + q)]);
#pragma unroll
    for (int q = 0; q < QB; ++q) dma16(srcB[q] + kt * KSTEP, &sB[st][64 * (QB * wave + q)]);
  };
  constexpr int PER_STAGE = QA + QB;              // vmcnt per stage and wave

  f32x4 acc[XT][YT];
#pragma unroll
  for (int x = 0; x < XT; ++x)
#pragma unroll
    for (int y = 0; y < YT; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wait until at most n stages of this wave's loads are still in flight
  // s_waitcnt immediate: vmcnt is 6 bits, [3:0] at bit 0 and [5:4] at bit 14;
  // expcnt and lgkmcnt at their maxima (no wait on them)
  auto wait_stages = [&](int n) {
    static_assert(2 * PER_STAGE <= 63, "vmcnt field");
    constexpr unsigned kRest = (7u << 4) | (15u << 8);
    constexpr unsigned kTwo = ((2 * PER_STAGE) & 15) | (((2 * PER_STAGE) >> 4) << 14) | kRest;
    constexpr unsigned kOne = (PER_STAGE & 15) | ((PER_STAGE >> 4) << 14) | kRest;
    if (n >= 2)
      __builtin_amdgcn_s_waitcnt(kTwo);
    else if (n == 1)
      __builtin_amdgcn_s_waitcnt(kOne);
    else
      __builtin_amdgcn_s_waitcnt(kRest);
  };
  auto read_frags = [&](int kt, f16x8 (&fa)[XT], f16x8 (&fb)[YT]) {
    const int st = kt % NS;
#pragma unroll
    for (int x = 0; x < XT; ++x) {
      const int row = wm * (TBM / WVM) + x * 16 + i;
      fa[x] = TL ? sA[st][(row >> 4) * 64 + lane] : sA[st][row * 4 + (g ^ lds_swz(row))];
    }
#pragma unroll
    for (int y = 0; y < YT; ++y) {
      const int row = wn * (TBN / WVN) + y * 16 + i;
      fb[y] = TL ? sB[st][(row >> 4) * 64 + lane] : sB[st][row * 4 + (g ^ lds_swz(row))];
    }
  };
  auto mma = [&](const f16x8 (&fa)[XT], const f16x8 (&fb)[YT]) {
#pragma unroll
    for (int x = 0; x < XT; ++x)
#pragma unroll
      for (int y = 0; y < YT; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[x], fb[y], acc[x][y], 0, 0, 0);
  };

#pragma unroll
  for (int k = 0; k < NS - 1; ++k)
    if (k < KT) issue(k);
  if constexpr (FP) {
    // Fragments of stage kt + 1 are read from LDS while the MFMAs of stage kt
    // run (two register sets).  The barrier of step kt publishes stage kt + 1
    // and ends every wave's MFMAs of step kt - 1, whose fragments were read a
    // step earlier, so stage kt - 1's buffer takes the loads of kt + NS - 1.
    static_assert(NS >= 3, "one stage in flight beyond the one being read");
    f16x8 fa0[XT], fb0[YT], fa1[XT], fb1[YT];
    if (KT > 0) {
      wait_stages(min(NS - 2, KT - 1));
      stage_barrier();
      read_frags(0, fa0, fb0);
    }
    auto step = [&](int kt, const f16x8 (&fa)[XT], const f16x8 (&fb)[YT], f16x8 (&na)[XT], f16x8 (&nb)[YT]) {
      if (kt + 1 < KT) {
        wait_stages(min(NS - 3, KT - 2 - kt));
        stage_barrier();
        if (kt + NS - 1 < KT) issue(kt + NS - 1);
      }
      // unconditional (the last step re-reads its own stage, which stays
      // valid): behind a branch the compiler waited for every LDS read here
      read_frags(min(kt + 1, KT - 1), na, nb);
      mma(fa, fb);
      // issue order: the next stage's LDS reads spread between these MFMAs
      // (a batch of them ahead of the MFMAs made the compiler wait for all)
#pragma unroll
      for (int q = 0; q < XT + YT; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, (XT * YT) / (XT + YT + 1), 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                           // LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, XT * YT - (XT + YT) * ((XT * YT) / (XT + YT + 1)), 0);
    };
    for (int kt = 0; kt < KT; kt += 2) {
      step(kt, fa0, fb0, fa1, fb1);
      if (kt + 1 < KT) step(kt + 1, fa1, fb1, fa0, fb0);
    }
  } else {
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt done (this wave's loads; later stages may stay in flight)
    wait_stages(min(NS - 2, KT - 1 - kt));
    stage_barrier();                     // every wave's share of stage kt is in; stage kt - 1 is consumed
    if (kt + NS - 1 < KT) issue(kt + NS - 1);
    f16x8 fa[XT], fb[YT];
    read_frags(kt, fa, fb);
    mma(fa, fb);
  }
  }

  // acc[x][y]: lane (i, g) holds rows 4g..4g+3 of column i of MFMA tile (x, y)
  const int rw0 = m0 + wm * (TBM / WVM), cw0 = n0 + wn * (TBN / WVN);
  // The 256 x 256 tile's fp32 outputs through LDS, a quarter (64 rows) at a
  // time: each lane's acc holds 4 rows of one column, so direct writes (and
  // residual reads) were 4-byte accesses, 128 per lane.  Rows of 256 + 4
  // floats (the pad puts a lane group's 4 rows on different banks); then
  // every thread passes 8 row-contiguous float4 to emit(row, col, value).
  auto staged = [&](auto &&emit) {
    constexpr int RS = TBN + 4;
    float *st = reinterpret_cast<float *>(s_lds);
    static_assert(64 * RS * 4 <= NS * (TBM + TBN) * 64, "a quarter tile fits the stages");
    stage_barrier();               // every wave is done with the operand stages
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      // rows 64 qq .. 64 qq + 63 are held by the waves with wm = qq / 2 (x = 4 (qq % 2) .. + 3)
      if (wm == qq / 2) {
#pragma unroll
        for (int xx = 0; xx < 4; ++xx)
#pragma unroll
          for (int y = 0; y < YT; ++y)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              st[(xx * 16 + 4 * g + r) * RS + wn * 64 + y * 16 + i] = acc[4 * (qq % 2) + xx][y][r];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = tid + 512 * k;               // float4 e of the quarter: row e / 64, columns 4 (e % 64) ..
        const int lr = e >> 6, c4 = (e & 63) * 4;
        const int row = m0 + 64 * qq + lr, col = n0 + c4;
        if (row < a.M && col < a.N) emit(row, col, *reinterpret_cast<const float4 *>(&st[lr * RS + c4]));
      }
      __syncthreads();
    }
  };
  // Used for the residual add (its reads were the exposed part); plain
  // stores -- the q/k/v output, split-K slices -- measured no faster staged
  // (32 x 8192 q/k/v 49.5 -> 51.1 ms per prefill).
  constexpr bool kStageable = TBM == 256 && TBN == 256 && WVM == 2 && WVN == 4;
  if (gridDim.z > 1) {
    float *ws = a.ws + (int64_t)blockIdx.z * a.M * a.N;
#pragma unroll
    for (int x = 0; x < XT; ++x)
#pragma unroll
      for (int y = 0; y < YT; ++y) {
        const int col = cw0 + y * 16 + i;
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rw0 + x * 16 + 4 * g + r;
          if (row < a.M) ws[(int64_t)row * a.N + col] = acc[x][y][r];
        }
      }
    return;
  }
  if constexpr (EPI == Epi::SwiGLU) {
    f16 *out = (f16 *)a.act_out;
    if (kRowEpilogue && TBM == 256 && TBN == 256 && (a.ldo & 7) == 0 && (a.N / 2) % 8 == 0) {
      // the tile's 256 x 128 values of h through LDS (rows of 128 + 8 f16),
      // then written as 16-byte row pieces rather than 2-byte stores
      constexpr int HS = TBN / 2 + 8;
      f16 *sh = reinterpret_cast<f16 *>(s_lds);
      static_assert(TBM * HS * 2 <= NS * (TBM + TBN) * 64, "the h tile fits the stages");
      stage_barrier();             // every wave is done with the operand stages
#pragma unroll
      for (int x = 0; x < XT; ++x)
#pragma unroll
        for (int p = 0; p < YT / 2; ++p) {
          const int fl = wn * (TBN / WVN / 2) + p * GU_BLOCK + i;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gt = acc[x][2 * p][r] * a.scale, up = acc[x][2 * p + 1][r] * a.scale;
            sh[(wm * (TBM / WVM) + x * 16 + 4 * g + r) * HS + fl] = (f16)(silu_f(gt) * up);
          }
        }
      __syncthreads();
      constexpr int V8 = TBN / 2 / 8;              // 16-byte pieces per row
#pragma unroll
      for (int k = 0; k < TBM * V8 / (64 * WVM * WVN); ++k) {
        const int e = tid + 64 * WVM * WVN * k;
        const int lr = e / V8, v = e % V8;
        const int row = m0 + lr, f = n0 / 2 + 8 * v;
        if (row < a.M && f < a.N / 2)
          *reinterpret_cast<f16x8 *>(out + (a.h_tiled ? tile_off(row, f, a.ldo) : (int64_t)row * a.ldo + f)) =
              *reinterpret_cast<const f16x8 *>(&sh[lr * HS + 8 * v]);
      }
    } else {
#pragma unroll
    for (int x = 0; x < XT; ++x)
#pragma unroll
      for (int p = 0; p < YT / 2; ++p) {
        const int f = cw0 / 2 + p * GU_BLOCK + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rw0 + x * 16 + 4 * g + r;
          if (row < a.M && f < a.N / 2) {
            const float gt = acc[x][2 * p][r] * a.scale, up = acc[x][2 * p + 1][r] * a.scale;
            out[a.h_tiled ? tile_off(row, f, a.ldo) : (int64_t)row * a.ldo + f] = (f16)(silu_f(gt) * up);
          }
        }
      }
    }
  } else if (EPI == Epi::ResidAdd && kStageable && kRowEpilogue && (a.ldo & 3) == 0 && a.N % 4 == 0) {
    staged([&](int row, int col, float4 v) {
      float4 *o = reinterpret_cast<float4 *>(a.out_f32 + (int64_t)row * a.ldo + col);
      float4 w = {v.x * a.scale, v.y * a.scale, v.z * a.scale, v.w * a.scale};
      if constexpr (EPI == Epi::ResidAdd) {
        const float4 x = *o;
        w.x += x.x;
        w.y += x.y;
        w.z += x.z;
        w.w += x.w;
      }
      *o = w;
    });
  } else {
#pragma unroll
    for (int x = 0; x < XT; ++x)
#pragma unroll
      for (int y = 0; y < YT; ++y) {
        const int col = cw0 + y * 16 + i;
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rw0 + x * 16 + 4 * g + r;
          if (row >= a.M) continue;
          float *o = a.out_f32 + (int64_t)row * a.ldo + col;
          const float v = acc[x][y][r] * a.scale;
          if constexpr (EPI == Epi::ResidAdd)
            *o += v;
          else
            *o = v;
        }
      }
  }
}

// out = epilogue(sum over slices of ws[slice]), one thread per output value
template <Epi EPI>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs a, int S) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t slice = (int64_t)a.M * a.N;
  if constexpr (EPI == Epi::SwiGLU) {
    const int F = a.N / 2;
    if (idx >= (int64_t)a.M * F) return;
    const int row = (int)(idx / F), f = (int)(idx % F);
    const int cg = (f / GU_BLOCK) * 2 * GU_BLOCK + f % GU_BLOCK;
    float gt = 0.f, up = 0.f;
    for (int z = 0; z < S; ++z) {
      gt += a.ws[z * slice + (int64_t)row * a.N + cg];
      up += a.ws[z * slice + (int64_t)row * a.N + cg + GU_BLOCK];
    }
    ((f16 *)a.act_out)[a.h_tiled ? tile_off(row, f, a.ldo) : (int64_t)row * a.ldo + f] =
        (f16)(silu_f(gt * a.scale) * (up * a.scale));
  } else if constexpr (EPI == Epi::QkvRope) {
    // one thread per (row, column pair) of the unpermuted layout: pair p is
    // dims d and d + hd/2 of head slot p / (hd/2) (q heads, then k, then v)
    const int half = a.qr.head_dim >> 1, npairs = a.N / 2;
    if (idx >= (int64_t)a.M * npairs) return;
    const int row = (int)(idx / npairs), p = (int)(idx % npairs);
    const int oc_lo = (p / half) * a.qr.head_dim + p % half, oc_hi = oc_lo + half;
    float lo = 0.f, hi = 0.f;
    for (int z = 0; z < S; ++z) {
      lo += a.ws[z * slice + (int64_t)row * a.N + oc_lo];
      hi += a.ws[z * slice + (int64_t)row * a.N + oc_hi];
    }
    int b, pos;
    qkv_row_pos(a.qr, row, b, pos);
    qkv_rope_store(a.qr, row, b, pos, oc_lo, oc_hi, lo * a.scale, hi * a.scale);
  } else {
    // four consecutive columns per thread (N and ldo are multiples of 4)
    const int64_t i4 = idx * 4;
    if (i4 >= slice) return;
    const int row = (int)(i4 / a.N), col = (int)(i4 % a.N);
    float4 v = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < S; ++z) {
      const float4 w = *reinterpret_cast<const float4 *>(a.ws + z * slice + i4);
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    float4 *o = reinterpret_cast<float4 *>(a.out_f32 + (int64_t)row * a.ldo + col);
    float4 r = {v.x * a.scale, v.y * a.scale, v.z * a.scale, v.w * a.scale};
    if constexpr (EPI == Epi::ResidAdd) {
      const float4 x = *o;
      r.x += x.x;
      r.y += x.y;
      r.z += x.z;
      r.w += x.w;
    }
    *o = r;
  }
}

}  // namespace

constexpr bool kLdsPipeline = true;
// stages of the 256 x 256 kernel (32 KB of LDS each); five (all 160 KB)
// measured slower: 32 x 8192 gate/up 393.4 -> 397.9 ms per prefill
constexpr int kBigStages = 4;
// 256 x 256 tiles halve the operand bytes per FLOP.  One workgroup runs per
// CU, so they pay once there are enough of them to fill the chip a few times
// over: with at least 512 tiles K is not split; with 192 .. 511 tiles (the
// N = H projections of a long prefill) K is split in two (three rounds of 256
// instead of one and a half), as long as each slice keeps 24 K tiles.
// Returns the K slices for the 256 x 256 kernel, or 0 where it is not used.
static int big_tile_splits(int M, int N, int K) {
  if (!kLdsPipeline || K % LK) return 0;
  const int big = ((M + 255) / 256) * ((N + 255) / 256);
  if (big >= 512) return 1;
  if (big >= 192 && K / LK >= 48) return 2;
  return 0;
}

int gemm_mfma_splits(int M, int N, int K) {
  if (N % 4) return 1;                           // the reduce takes four columns per thread
  if (const int bs = big_tile_splits(M, N, K)) return bs;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles >= 128) return 1;
  int S = (256 + tiles - 1) / tiles;
  const int max_s = ((K + BK - 1) / BK) / 2;     // at least two K tiles per slice
  if (S > max_s) S = max_s;
  if (S > 16) S = 16;
  return S < 1 ? 1 : S;
}

bool gemm_mfma_supported(const GemmArgs &a) {
  if (a.epi == Epi::QkvRope && (a.N % 2 || a.qr.head_dim % 2 || gemm_mfma_splits(a.M, a.N, a.K) < 2)) return false;
  return (a.K % 8) == 0 && (a.lda % 8) == 0 && (a.epi != Epi::SwiGLU || a.N % 128 == 0);
}

hipError_t launch_gemm_mfma(hipStream_t s, const GemmArgs &a) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!gemm_mfma_supported(a)) return hipErrorInvalidValue;
  const int S = (a.splits > 1 && a.ws && a.N % 4 == 0 && (a.ldo % 4 == 0 || a.epi == Epi::QkvRope)) ? a.splits : 1;
  // QkvRope runs split only: the multiply writes raw slices (any epilogue's
  // kernel does), and the reduction applies bias + RoPE + the writes
  if (a.epi == Epi::QkvRope && S < 2) return hipErrorInvalidValue;
  // unit-tiled A and W only on the LDS-pipeline kernels (K % 32 == 0); h
  // written tiled only by a SwiGLU epilogue with N / 2 % 32 == 0
  if ((a.tiled && !(kLdsPipeline && a.K % LK == 0)) || (a.h_tiled && (a.epi != Epi::SwiGLU || (a.N / 2) % 32)))
    return hipErrorInvalidValue;
  const Epi ke = a.epi == Epi::QkvRope ? Epi::StoreF32 : a.epi;
  const int tiles = ((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  dim3 grid(8 * ((tiles + 7) / 8), 1, S);
  if (big_tile_splits(a.M, a.N, a.K) > 0) {
    const int big = ((a.N + 255) / 256) * ((a.M + 255) / 256);
    dim3 g2(8 * ((big + 7) / 8), 1, S);
    // four stages, the next stage's fragments read from LDS during this
    // stage's MFMAs: gate/up of an 8x2048 prefill 25.5 -> 24.3 ms (three
    // stages with the same pipelining: 26.1 ms)
    switch (ke) {
      case Epi::StoreF32:
        if (a.tiled) QW_LAUNCH((gemm_lds_kernel<Epi::StoreF32, 256, 256, 2, 4, kBigStages, true, true>), dim3(g2), dim3(512), 0, s, a);
        else QW_LAUNCH((gemm_lds_kernel<Epi::StoreF32, 256, 256, 2, 4, kBigStages, true>), dim3(g2), dim3(512), 0, s, a);
        break;
      case Epi::ResidAdd:
        if (a.tiled) QW_LAUNCH((gemm_lds_kernel<Epi::ResidAdd, 256, 256, 2, 4, kBigStages, true, true>), dim3(g2), dim3(512), 0, s, a);
        else QW_LAUNCH((gemm_lds_kernel<Epi::ResidAdd, 256, 256, 2, 4, kBigStages, true>), dim3(g2), dim3(512), 0, s, a);
        break;
      case Epi::SwiGLU:
        if (a.tiled) QW_LAUNCH((gemm_lds_kernel<Epi::SwiGLU, 256, 256, 2, 4, kBigStages, true, true>), dim3(g2), dim3(512), 0, s, a);
        else QW_LAUNCH((gemm_lds_kernel<Epi::SwiGLU, 256, 256, 2, 4, kBigStages, true>), dim3(g2), dim3(512), 0, s, a);
        break;
    }
  } else if (kLdsPipeline && a.K % LK == 0) {
    switch (ke) {
      case Epi::StoreF32:
        if (a.tiled) QW_LAUNCH((gemm_lds_kernel<Epi::StoreF32, 128, 128, 2, 2, 4, false, true>), dim3(grid), dim3(256), 0, s, a);
        else QW_LAUNCH((gemm_lds_kernel<Epi::StoreF32, 128, 128, 2, 2, 4>), dim3(grid), dim3(256), 0, s, a);
        break;
      case Epi::ResidAdd:
        if (a.tiled) QW_LAUNCH((gemm_lds_kernel<Epi::ResidAdd, 128, 128, 2, 2, 4, false, true>), dim3(grid), dim3(256), 0, s, a);
        else QW_LAUNCH((gemm_lds_kernel<Epi::ResidAdd, 128, 128, 2, 2, 4>), dim3(grid), dim3(256), 0, s, a);
        break;
      case Epi::SwiGLU:
        if (a.tiled) QW_LAUNCH((gemm_lds_kernel<Epi::SwiGLU, 128, 128, 2, 2, 4, false, true>), dim3(grid), dim3(256), 0, s, a);
        else QW_LAUNCH((gemm_lds_kernel<Epi::SwiGLU, 128, 128, 2, 2, 4>), dim3(grid), dim3(256), 0, s, a);
        break;
    }
  } else switch (ke) {
    case Epi::StoreF32: QW_LAUNCH((gemm_mfma_kernel<Epi::StoreF32>), dim3(grid), dim3(256), 0, s, a); break;
    case Epi::ResidAdd: QW_LAUNCH((gemm_mfma_kernel<Epi::ResidAdd>), dim3(grid), dim3(256), 0, s, a); break;
    case Epi::SwiGLU: QW_LAUNCH((gemm_mfma_kernel<Epi::SwiGLU>), dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int64_t n = (a.epi == Epi::SwiGLU || a.epi == Epi::QkvRope) ? (int64_t)a.M * (a.N / 2)
                                                                     : (int64_t)a.M * a.N / 4;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  switch (a.epi) {
    case Epi::StoreF32: splitk_reduce_kernel<Epi::StoreF32><<<blocks, 256, 0, s>>>(a, S); break;
    case Epi::ResidAdd: splitk_reduce_kernel<Epi::ResidAdd><<<blocks, 256, 0, s>>>(a, S); break;
    case Epi::SwiGLU: splitk_reduce_kernel<Epi::SwiGLU><<<blocks, 256, 0, s>>>(a, S); break;
    case Epi::QkvRope: splitk_reduce_kernel<Epi::QkvRope><<<blocks, 256, 0, s>>>(a, S); break;
  }
  return hipGetLastError();
}

}  // namespace qw
