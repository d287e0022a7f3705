// Internal declarations shared by the HIP kernels and the host runtime of
// libqw.so.  Device helpers are header-inline; every kernel family has a host
// launcher declared here and defined next to its kernel.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qw {

// Kernel-duration timing.  While `launch_timing` holds an event pair, the
// launches of the timed kernel families pass it to hipExtLaunchKernelGGL,
// which records the events at the start and at the end of the kernel itself
// (no dispatch gap inside the interval), on the kernel's own stream.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchTiming launch_timing;

#define QW_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                                   \
  do {                                                                                                     \
    if (::qw::launch_timing.start)                                                                         \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, ::qw::launch_timing.start,                  \
                            ::qw::launch_timing.stop, 0, __VA_ARGS__);                                     \
    else                                                                                                   \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                                 \
  } while (0)

// Packed gate/up projection: rows of W_gate and W_up alternate in blocks of
// GU_BLOCK rows ([g0..g15, u0..u15, g16..g31, u16..u31, ...]), so a tile of
// whole block pairs holds the gate and up value of the same features.
constexpr int GU_BLOCK = 16;

typedef _Float16 f16;

// Bits of a model's status word on the device.  Kernels set them with
// atomicOr; qw_check_ids and qw_check_numerics read and clear them.
constexpr int kFlagBadId = 1;       // a token id outside [0, V) was read as id 0
constexpr int kFlagNonFinite = 2;   // a logit of a greedy row was inf or NaN
constexpr int kFlagFixRange = 4;    // a fixed-point addend of the decode residual or sums exceeded 2^23

// The calling thread's qw_last_error message: report() sets it and returns
// `st`; clear_error() empties it (every entry point starts with it).
int report(int st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// ------------------------------------------------------------ device helpers
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }  // RNE

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// One 16-byte-per-lane load straight into LDS at the wave-uniform address
// `lds` (+ 16 * lane).  Issued as assembly so that the compiler does not
// drain every load in flight before each LDS read it cannot prove disjoint
// from it; completion is awaited explicitly (s_waitcnt vmcnt) before the
// barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void *src, const void *lds) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);   // wave-uniform
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0v) : "memory");
}
// s_barrier without the release/acquire fences __syncthreads carries (the
// waits they imply are issued explicitly); the empty asm keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// s_waitcnt with vmcnt = n (6 bits: [3:0] at bit 0, [5:4] at bit 14) and no
// wait on expcnt or lgkmcnt
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ------------------------------------------------------------ KV cache layout
// Positions of a sequence are grouped in blocks of kKvBlock.  Dense layout
// (table == NULL): a layer's cache is [max_batch][nkv][max_seq][hd].  Paged
// layout: a layer's cache is a pool [num_blocks][nkv][kKvBlock][hd], and
// table[b * blocks_per_seq + p] names the pool block that holds positions
// kKvBlock p .. kKvBlock p + kKvBlock - 1 of sequence b.
constexpr int kKvBlock = 64;

struct KvMap {
  const int *table = nullptr;  // paged: [max_batch][blocks_per_seq]; NULL: dense
  int blocks_per_seq = 0;
  int max_seq = 0;             // dense: positions per sequence
};

// Element offset of (sequence b, KV head j, position pos) from a layer's base.
__device__ __forceinline__ int64_t kv_offset(const KvMap &m, int nkv, int hd, int b, int j, int pos) {
  if (m.table) {
    const int blk = m.table[b * m.blocks_per_seq + (pos / kKvBlock)];
    return (((int64_t)blk * nkv + j) * kKvBlock + (pos % kKvBlock)) * hd;
  }
  return (((int64_t)b * nkv + j) * m.max_seq + pos) * hd;
}

// Ragged batches: sequence s holds rows cu[s] .. cu[s+1]-1 of the packed
// prompt rows; its transposed V copy starts at pcu[s] * nkv * hd elements,
// pcu being the prefix sums of round_up(length, kKvBlock).
struct RaggedRows {
  const int *cu = nullptr;     // [n + 1], or NULL for equal-length sequences
  const int *pcu = nullptr;    // [n + 1]
  int n = 0;
};

// The sequence of packed row t (cu[s] <= t < cu[s+1]).
__device__ __forceinline__ int ragged_seq(const int *cu, int n, int t) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------ launch params
enum class Epi : int {
  StoreF32 = 0,   // out_f32[m, n] = acc * scale
  ResidAdd = 1,   // resid[m, n] += acc * scale
  SwiGLU = 2,     // act_out[m, f] = silu(gate) * up over GU_BLOCK-interleaved rows
  QkvRope = 3,    // prefill q/k/v projection (split K only): + bias, RoPE on q and k, q to q_out, k and v into the cache
};

// The prefill q/k/v projection's epilogue (Epi::QkvRope), applied by the
// split-K reduction (the projection must run split): rows are prompt rows
// from position 0 (rows_per_seq each, or the ragged sequences of rag).
struct QkvRopeArgs {
  const float *bias = nullptr;    // [nq*hd + 2*nkv*hd], by column of the unpermuted layout
  const float2 *rope = nullptr;   // [max_seq, hd/2] (cos, sin)
  void *q_out = nullptr;          // [M, nq*hd] f16
  void *k_cache = nullptr, *v_cache = nullptr;   // layer base
  KvMap kv;
  RaggedRows rag;
  int rows_per_seq = 0, n_heads = 0, n_kv_heads = 0, head_dim = 0;
};

struct GemmArgs {
  const void *A;        // [M, K] activations (compute type), row stride lda
  const void *W;        // [N, K] weights (compute type), row stride K
  int M, N, K, lda;
  float scale;          // exact power of two undoing the weight scaling
  Epi epi;
  float *out_f32;       // StoreF32: [M, ldo]; ResidAdd: residual [M, ldo]
  void *act_out;        // SwiGLU: [M, ldo] compute type, ldo = N / 2
  int ldo;
  int splits = 1;       // MFMA path: K slices (> 1 needs ws)
  float *ws = nullptr;  // [splits, M, N] fp32 slice tiles
  QkvRopeArgs qr;       // QkvRope
  int tiled = 0;        // A and W unit-tiled (W = the tiled weight copy; A rows padded to 16)
  int h_tiled = 0;      // SwiGLU: h written unit-tiled (the down projection's A)
};

struct RopeCacheArgs {
  const float *qkv;      // [T, nq*hd + 2*nkv*hd] projections without bias
  const float *bias;     // [nq*hd + 2*nkv*hd]
  const float2 *rope;    // [max_seq, hd/2] (cos, sin)
  void *q_out;           // [T, nq*hd] compute type
  void *k_cache, *v_cache;  // layer base (layout: kv)
  KvMap kv;
  RaggedRows rag;        // rag.cu set: sequence s is rows cu[s] .. cu[s+1]-1 from position 0
  int T, rows_per_seq, n_heads, n_kv_heads, head_dim;
  int pos0;              // position of each sequence's first row ...
  const int *pos0_dev;   // ... or, if non-null, pos0_dev[b] for sequence b
};

struct AttnArgs {
  const void *q;              // [T, nq*hd]
  const void *k_cache, *v_cache;  // layer base (layout: kv)
  KvMap kv;
  RaggedRows rag;             // as in RopeCacheArgs
  const int *tiles;           // ragged prefill: (sequence << 16 | query tile) work list, or NULL
  int n_tiles;
  const void *v_t;            // prefill (f16): V of the prompt transposed, [B][nkv][hd][round_up(P, 64)]
  void *o;                    // [T, nq*hd]
  int o_tiled = 0;            // prefill (f16): o unit-tiled (the o projection's operand)
  int T, rows_per_seq, n_heads, n_kv_heads, head_dim;
  int pos0;
  const int *pos0_dev;        // pos0_dev[b] for sequence b
  float softmax_scale;
};

// Unit-tiled layout of f16 GEMM operands (the weight copies, and u, o and h
// of prefill and of the batched decode step): a [rows, K] matrix as 1 KB
// tiles of 16 rows x 32 k, tile (R, U) =
// rows 16R .. 16R + 15, k 32U .. 32U + 31, tiles of a row block consecutive
// in U; inside a tile, element (i, k) at 128 ((k % 32) / 8) + 8 i + k % 8, the
// lane order of the MFMA operand (lane i + 16 g holds row i, k 8g .. 8g + 7),
// so one wave-wide 16-byte load reads one tile.  Rows are padded to a multiple
// of kTileRows for weights and of 16 for activations.
constexpr int kTileRows = 64;
__device__ __host__ __forceinline__ int64_t tile_off(int row, int k, int K) {
  return ((int64_t)(row >> 4) * (K >> 5) + (k >> 5)) * 512 + ((k & 31) >> 3) * 128 + (row & 15) * 8 + (k & 7);
}

// RMSNorm hand-off between the batched decode projections (more than two
// rows), see k_decode.hip.  The projection that finishes a block of residual
// columns writes the next projection's operand without the row scale,
// u = f16(x * w), and the block's sum of x^2 per row; the projection that
// reads u multiplies each output row by 1/rms of its row.
constexpr int kNormPartsMax = 128;     // sums of squares per row (column blocks of the producer)
constexpr int kSyncCounters = 256;     // last-arrival counters of one decode step
struct RowNormOut {
  const float *w;           // norm weight [N] of the consumer; NULL: no hand-off
  void *u;                  // f16 [M, N]
  float *ss;                // [M, ss_ld]: column block c's sum of x^2 at column c
  int ss_ld;
  int *counters;            // one per column block, zero between launches
  int64_t rep_stride;       // residual replicas of out_fix (value = their sum)
  int tiled;                // u in the unit-tiled layout
};
struct RowNormIn {
  const float *ss;          // NULL: the operand is already normalised
  int ss_ld, parts;         // parts <= kNormPartsMax sums per row
  float dim, eps;           // H and the RMSNorm epsilon
};

// Decode-step projection (B <= 32 rows), see k_decode.hip.  f16 operands.
struct DecGemvArgs {
  const void *W;            // [N, K] f16
  int M, N, K;
  int act_mode;             // 0: f16 act; 1: RMSNorm of x_fix; 2: silu(gate)*up of act_fix;
                            // 3: merge of split-KV attention partials
  const void *act;          // mode 0: [M, lda] f16
  const long long *x_fix;   // mode 1: [M, lda] fixed-point residual rows (lda = K), stored as
  int64_t x_rep_stride;     //   kXReps replicas x_rep_stride apart whose sum is the value
  const float *norm_w;      // mode 1: [K]
  float eps;                // mode 1
  const long long *act_fix; // mode 2: [M, lda] fixed-point gate/up sums (lda = 2K)
  const float *part_m, *part_l, *part_o;  // mode 3: [M][n_heads][S] (+ [head_dim])
  int attn_splits, n_heads, head_dim;     // mode 3
  int lda;
  float scale;              // exact power of two undoing the weight scaling
  long long *out_fix;       // fixed-point accumulator [M, ldo] (atomic adds)
  int ldo;
  int splits;               // K slices
  int units_per_split;      // set by the launcher
  long long *clear;         // side job: zero clear[0 .. clear_n) (may be NULL)
  int64_t clear_n;
  int role_gate_up;          // 1 for the gate/up projection (separate kernel symbol in profiles)
  // gate/up without a K split: silu(gate) * up of the GU_BLOCK-interleaved rows
  // written as f16 h [M, ldh] (no fixed-point output)
  int swiglu_out;
  void *h_out;
  int ldh;
  // LM-head mode: logits [M, ldo] (may be NULL) and per-64-row-block argmax
  int logits_mode;
  float *logits;
  float *arg_v;             // [M, ceil(N / 64)]
  int *arg_i;
  int *num_flag;            // status word (kFlagFixRange, kFlagNonFinite)
  RowNormOut nout;          // batched FixAdd residual projections: the next norm's operand
  RowNormIn nin;            // batched projections and the LM head: operand u without 1/rms
  int w_tiled;              // W in the unit-tiled layout (rows padded to kTileRows)
  int act_tiled;            // batched projections: f16 operand (and a SwiGLU projection's h) unit-tiled
};

// Decode-step attention, see k_decode.hip.
struct DecAttnArgs {
  const long long *qkv_fix;          // [batch, nq*hd + 2*nkv*hd] fixed-point projection sums
  const float *bias;                 // [nq*hd + 2*nkv*hd]
  const float2 *rope;                // [max_seq, hd/2]
  void *k_cache, *v_cache;           // layer base (layout: kv)
  KvMap kv;
  void *o;                           // splits == 1: [batch, nq*hd] f16
  float *part_m, *part_l, *part_o;   // splits > 1: [batch][nq][splits] (+ [hd])
  int splits;
  int head_parallel;                 // 1: waves split the heads (short contexts), 0: waves split the keys
  int batch, n_heads, n_kv_heads, head_dim;
  const int *pos_dev;                // pos_dev[b]: position of row b's new token
  float softmax_scale;
  long long *clear;                  // side job: zero clear[0 .. clear_n)
  int64_t clear_n;
  int o_tiled;                       // splits == 1: o in the unit-tiled layout
};

// Decode-step attention merged with the o projection, for one or two rows and
// short contexts, see k_decode.hip.  Adds o . W_o^T (scaled) into x_out.
struct DecAttnOArgs {
  const long long *qkv_fix;          // [batch, nq*hd + 2*nkv*hd] fixed-point projection sums
  const float *bias;                 // [nq*hd + 2*nkv*hd]
  const float2 *rope;                // [max_seq, hd/2]
  void *k_cache, *v_cache;           // layer base (layout: kv)
  KvMap kv;
  int batch, n_heads, n_kv_heads, head_dim;
  const int *pos_dev;                // pos_dev[b]: position of row b's new token
  float softmax_scale;
  const void *w_o;                   // [H, nq*hd] f16
  const void *w_o_tl;                // w_o unit-tiled (read instead of w_o when set)
  float o_scale;
  int H;
  long long *x_out;                  // [batch, H] fixed-point residual (atomic adds)
  long long *clear;                  // side job: zero clear[0 .. clear_n)
  int64_t clear_n;
  int *num_flag;                     // status word (kFlagFixRange)
};
bool dec_attn_o_supported(int head_dim, int hidden);

// The decode residual stream is kept as this many fixed-point replicas whose
// sum is the value: the fused MLP, whose workgroups would otherwise all add
// into the same addresses, spreads its atomics over them; every reader loads
// all replicas in one batch.
constexpr int kXReps = 2;

// Decode-step MLP for one or two rows, see k_decode.hip:
//   x_out = x_in + W_down . (silu(W_gate u) * (W_up u)),  u = RMSNorm(x_in) * norm_w
// x_out must be zero on entry (workgroup 0 adds x_in itself).
struct DecMlpArgs {
  const long long *x_in;             // [kXReps][M, H] fixed-point residual (read; value = sum of replicas)
  long long *x_out;                  // [kXReps][M, H] fixed-point residual (accumulated)
  int64_t rep_stride;                // elements between replicas; workgroup p adds into replica p % kXReps
  const float *norm_w;               // [H] post-attention norm weight
  float eps;
  const void *w_gu;                  // [2I, H] f16, GU_BLOCK-interleaved gate/up rows
  float gu_scale;
  const void *w_down_t;              // [I, H] f16, W_down transposed
  float down_scale;
  const void *w_gu_tiled;            // w_gu unit-tiled (read instead of w_gu when set)
  int M, H, I;
  long long *clear;                  // side job: zero clear[0 .. clear_n) (may be NULL)
  int64_t clear_n;
  int *num_flag;                     // status word (kFlagFixRange)
};
bool dec_mlp_supported(int hidden, int inter);

// ------------------------------------------------------------ launchers
// Each returns the hipError_t of its launch.  `f16_mode` selects the compute
// type (f16 when true, float when false).
// row r reads ids[(r / rows_per_seq) * ids_stride + r % rows_per_seq]
hipError_t launch_embed(hipStream_t s, bool f16_mode, const int32_t *ids, int rows, int rows_per_seq,
                        int64_t ids_stride, const void *emb, float emb_scale, int hidden, int vocab, float *x,
                        int *bad_id_flag);
// tiled: f16 out in the unit-tiled layout (hidden % 32 == 0, at most kRmsTiledMaxHidden)
constexpr int kRmsTiledMaxHidden = 4096;
hipError_t launch_rmsnorm(hipStream_t s, bool f16_mode, const float *x, int rows, int row_stride,
                          int hidden, const float *w, float eps, void *out, bool tiled = false);
hipError_t launch_rope_cache(hipStream_t s, bool f16_mode, const RopeCacheArgs &a);
hipError_t launch_attention_generic(hipStream_t s, bool f16_mode, const AttnArgs &a);
bool attn_prefill_supported(int head_dim);
int attn_prefill_query_tile();     // queries per workgroup (a ragged tile list counts in these)
hipError_t launch_attention_prefill(hipStream_t s, const AttnArgs &a);   // f16, prompt from position 0
// v_t[b][j][d][t] = V cache[b][j][t][d] for t < P, 0 for P <= t < round_up(P, 64);
// with rag.cu set, sequence s (length cu[s+1] - cu[s]) at pcu[s] * nkv * hd,
// its rows round_up(length, 64) long; max_len bounds the lengths
hipError_t launch_transpose_v(hipStream_t s, const void *v_cache, const KvMap &kv, const RaggedRows &rag, int B,
                              int n_kv_heads, int head_dim, int P, int max_len, void *v_t);
hipError_t launch_gemm_generic(hipStream_t s, bool f16_mode, const GemmArgs &a);
bool gemm_mfma_supported(const GemmArgs &a);
int gemm_mfma_splits(int M, int N, int K);
hipError_t launch_gemm_mfma(hipStream_t s, const GemmArgs &a);     // f16 operands
bool decode_fast_supported(int head_dim, int group, int hidden, int q_dim, int inter);
int dec_gemv_splits(int N, int K, int M, int target_groups);
int dec_attn_splits(int batch, int n_kv_heads, int ctx, int target_groups);
// with nout.w set, also u = f16(x * w) and each row's sum of x^2 (nout.ss[b * ss_ld])
hipError_t launch_dec_embed(hipStream_t s, const int32_t *ids, int B, const void *emb, float emb_scale, int H, int V,
                            long long *x_fix, int *bad, long long *clr0, int64_t n0, long long *clr1, int64_t n1,
                            const RowNormOut &nout);
// the column blocks a batched FixAdd projection of N outputs hands its norm
// sums over (0: it cannot, and a norm kernel runs instead)
int dec_norm_parts(int M, int N, int K);
hipError_t launch_dec_norm(hipStream_t s, const long long *x_fix, int64_t rep_stride, int B, int H,
                           const float *w, float eps, void *u);
// also advances pos_dev[b] for every row b
hipError_t launch_dec_end(hipStream_t s, const float *arg_v, const int *arg_i, int nblk, int B, int32_t *next,
                          int *pos_dev);
hipError_t launch_dec_gemv(hipStream_t s, const DecGemvArgs &a);
hipError_t launch_dec_attention(hipStream_t s, const DecAttnArgs &a);
hipError_t launch_dec_mlp(hipStream_t s, const DecMlpArgs &a);
// the merged split-KV attention output o [B, nq*hd] as f16, formed once for
// batches of more than two rows
hipError_t launch_dec_merge(hipStream_t s, const float *pm, const float *pl, const float *po, int S, int B, int nq,
                            int hd, void *o, bool tiled = false);
// Wt = W [N, K] f16 in the unit-tiled layout, rows padded with zeros to a
// multiple of kTileRows (Wt holds round_up(N, kTileRows) * K elements)
hipError_t launch_tile_units(hipStream_t s, const void *W, int N, int K, void *Wt);
hipError_t launch_dec_attn_o(hipStream_t s, const DecAttnOArgs &a);
// also sets kFlagNonFinite in *flag when a row holds an inf or NaN logit, and
// adds pos_add to pos_dev[r] for every row r (when pos_dev is non-NULL)
hipError_t launch_argmax(hipStream_t s, const float *logits, int rows, int vocab, int64_t row_stride,
                         int32_t *next_ids, int *pos_dev, int pos_add, int *flag);
// dst[b * dst_stride + dst_col] = src[b] (and seq[b * seq_stride + seq_col] = src[b] if seq)
hipError_t launch_put_column(hipStream_t s, int32_t *dst, int64_t dst_stride, int dst_col, int32_t *seq,
                             int64_t seq_stride, int seq_col, const int32_t *src, int B);
// rows x n four-byte values from src (row stride src_stride) to dst (dst_stride)
hipError_t launch_copy_rows(hipStream_t s, void *dst, int64_t dst_stride, const void *src, int64_t src_stride,
                            int rows, int64_t n);
hipError_t launch_copy_i32(hipStream_t s, int32_t *dst, const int32_t *src, int n);
// next_dst[0..b) = next_src; if logits_dst, logits_dst[0..n_logits) = logits_src
hipError_t launch_stage_out(hipStream_t s, int32_t *next_dst, const int32_t *next_src, int b, float *logits_dst,
                            const float *logits_src, int64_t n_logits);

// Sampling of the next token from B rows of logits (row stride row_stride)
// by the counter-based draw for n = pos_dev[b] tokens before it in row b; with finished
// non-NULL the end-of-sequence rule for `eos` applies.  See k_sample.hip.
hipError_t launch_sample(hipStream_t s, const float *logits, int64_t row_stride, int B, int V, float temperature,
                         int top_k, float top_p, uint64_t seed, const int *pos_dev, int32_t *next, int *finished,
                         int eos);
hipError_t launch_eos(hipStream_t s, int32_t *next, int *finished, int eos, int B);
hipError_t launch_fill_int(hipStream_t s, int *p, int v, int n);

// Small host-to-device updates carried in the kernel arguments (nothing is
// staged in host memory, so later host changes cannot race the copy):
// dst[idx[k]] = val[k] for k < n, in launches of up to kPutChunk pairs.
constexpr int kPutChunk = 240;
hipError_t launch_put_ints(hipStream_t s, int *dst, const int *idx, const int *val, int n);
// the last row of each ragged sequence: dst[k * H + c] = src[(cu[k+1] - 1) * H + c]
// for k < n, c < H (fp32; cu on the device)
hipError_t launch_gather_last_rows(hipStream_t s, float *dst, const float *src, const int *cu, int n, int H);

// set-up kernels (qw_create); src_kind is the storage type of the caller's
// weights
constexpr int kWeightF32 = 0, kWeightBF16 = 1, kWeightF16 = 2;
hipError_t launch_absmax(hipStream_t s, int src_kind, const void *src, int64_t n, unsigned *out_bits);
// dst[dst_offset + i] = src[i] * scale for i < n (scale: exact power of two)
hipError_t launch_convert(hipStream_t s, int src_kind, const void *src, int64_t n, bool dst_f16, void *dst,
                          int64_t dst_offset, float scale);
hipError_t launch_convert_gu(hipStream_t s, int src_kind, const void *gate, const void *up, int inter,
                             int hidden, bool dst_f16, void *dst, float scale);
hipError_t launch_convert_t(hipStream_t s, int src_kind, const void *src, int rows, int cols, void *dst,
                            float scale);   // f16 dst[cols][rows]

hipError_t launch_rope_table(hipStream_t s, float2 *table, int max_seq, int head_dim, double theta);

}  // namespace qw
