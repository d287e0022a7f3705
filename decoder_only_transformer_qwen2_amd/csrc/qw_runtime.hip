// Host runtime of libqw.so: argument and state validation, the library's own
// packed weight copies, KV cache and workspace, the per-layer launch sequence
// of prefill and decode, and the captured HIP graph of a decode step.
//
// Launch sequence of one decoder block (pre-norm, "LLM Speedrun:
// Architecture", section "Why pre-norm over post-norm?"; "augur": decoder
// blocks are norm, attention, residual, norm, MLP, residual):
//   rmsnorm(x) -> u;  u.Wqkv^T -> qkv;  bias + RoPE -> q, cache[k, v];
//   attention(q, cache) -> o;  x += o.Wo^T;  rmsnorm(x) -> u;
//   silu(u.Wg^T) * (u.Wu^T) -> h;  x += h.Wd^T
// then, after the last block, the final norm of each sequence's last row, the
// LM head and the greedy argmax ("augur": full forward pass; greedy
// generation).  Prefill runs this over every prompt row at once; a decode step
// over one row per sequence at the next position ("Building a Qwen2.5-1.5B
// Inference Engine From Scratch", section 1: prefill and decode).
#include "../../include/qw.h"
#include "qw_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

using namespace qw;

namespace qw {
thread_local LaunchTiming launch_timing;
}

namespace {
thread_local std::string g_err;
}

namespace qw {
int report(int st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
void clear_error() { g_err.clear(); }
}  // namespace qw

namespace {

#define fail(ST, ...) ((qw_status)::qw::report((ST), __VA_ARGS__))

#define HIP_TRY(expr)                                                                         \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess)                                                                     \
      return fail(e_ == hipErrorOutOfMemory ? QW_ERR_OUT_OF_MEMORY : QW_ERR_HIP, "%s: %s (%s:%d)", \
                  #expr, hipGetErrorString(e_), __FILE__, __LINE__);                          \
  } while (0)

enum Family { F_EMBED, F_RMSNORM, F_GEMM_QKV, F_ROPE_CACHE, F_ATTENTION, F_GEMM_O, F_GEMM_GATE_UP,
              F_GEMM_DOWN, F_LM_HEAD, F_ARGMAX, F_MLP, F_ATTN_O, F_ATTN_MERGE, F_COUNT };
const char *const kFamilyNames[] = {"embed",  "rmsnorm",      "gemm_qkv",  "rope_cache", "attention", "gemm_o",
                                    "gemm_gate_up", "gemm_down", "lm_head", "argmax", "mlp", "attn_o",
                                    "attn_merge"};
static_assert(sizeof(kFamilyNames) / sizeof(kFamilyNames[0]) == F_COUNT, "one name per kernel family");
const char *const kFamilyList =
    "embed,rmsnorm,gemm_qkv,rope_cache,attention,gemm_o,gemm_gate_up,gemm_down,lm_head,argmax,mlp,attn_o,"
    "attn_merge";

struct LayerBuf {
  void *w_qkv = nullptr;    // [qd + 2 kvd, H]
  float *b_qkv = nullptr;   // [qd + 2 kvd]
  void *w_o = nullptr;      // [H, qd]
  void *w_gu = nullptr;     // [2I, H], GU_BLOCK-interleaved
  void *w_down = nullptr;   // [H, I]
  void *w_down_t = nullptr; // [I, H] copy read by the fused decode MLP (f16 mode)
  // unit-tiled copies of w_qkv, w_o, w_gu, w_down (f16 models whose widths
  // are multiples of 32), read by the prefill GEMMs and the decode projections
  void *tl_qkv = nullptr, *tl_o = nullptr, *tl_gu = nullptr, *tl_down = nullptr;
  float *in_norm = nullptr, *post_norm = nullptr;
  float s_qkv = 1.f, s_o = 1.f, s_gu = 1.f, s_down = 1.f;
};

}  // namespace

// Per-step buffers of qw_decode_step_noalloc: one static array per GPU,
// held until the process ends.  In host code `scratch` is only a handle for
// hipGetSymbolAddress; its device address (one per GPU) is looked up once
// per device when the first model is created there and kept in
// g_scratch_dev, which is what kernels receive.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static_assert(kNoAllocScratchBytes == QW_NOALLOC_SCRATCH_BYTES, "the header states the array's size");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];
}  // namespace

struct qw_model {
  qw_config cfg{};
  int device = 0;            // HIP device the model lives on
  bool f16 = false;          // compute type: f16 (bf16 weights) or f32
  size_t esz = 4;
  int qd = 0, kvd = 0, nqkv = 0;
  int64_t rows_cap = 0;      // max_batch * max_seq
  hipStream_t stream = nullptr;
  hipStream_t cap = nullptr;
  std::vector<LayerBuf> L;
  void *emb = nullptr;
  float emb_scale = 1.f;
  void *head = nullptr;
  void *head_tl = nullptr;           // head unit-tiled (every LM head), rows padded to kTileRows
  float head_scale = 1.f;
  float *final_norm = nullptr;
  void *k_cache = nullptr, *v_cache = nullptr;
  int64_t cache_layer_elems = 0;
  // Paged cache (qw_create_paged): each layer's cache is a pool of num_blocks
  // blocks of kKvBlock positions, and block_table[b][p] names the block that
  // holds positions kKvBlock p .. of sequence b.  The host keeps the free list
  // and each sequence's blocks; blocks are handed out as sequences reach them
  // (prefill: the prompt's; decode: one more every kKvBlock steps) and all
  // return to the pool when a prefill starts a new batch.
  bool paged = false;
  int num_blocks = 0, blocks_per_seq = 0;
  int *block_table = nullptr;                  // device [max_batch][blocks_per_seq]
  std::vector<int> free_blocks;                // popped from the back
  std::vector<std::vector<int>> seq_blocks;    // [max_batch] blocks in position order
  // tokens each sequence holds (host mirror of pos_dev; ragged batches differ)
  std::vector<int> pos_host;
  // ragged prefill: cu [max_batch + 1], pcu [max_batch + 1], query-tile list
  int *rag_meta = nullptr;
  int rag_tiles_cap = 0;
  float *x_last = nullptr;                     // [max_batch, H] last rows of a ragged prefill
  float2 *rope = nullptr;
  float *x = nullptr, *qkv = nullptr, *logits = nullptr;
  void *u = nullptr, *q = nullptr, *o = nullptr, *h = nullptr;
  int *pos_dev = nullptr;
  int *status = nullptr;     // status word: kFlagBadId | kFlagNonFinite | kFlagFixRange
  int32_t *ids_stage = nullptr, *next_stage = nullptr;   // [max_batch] rows the decode graph reads / writes
  int32_t *seq_ids = nullptr;        // [max_batch][max_seq] sequences of the uncached generation
  // sampling instead of the greedy choice (qw_set_sampling) and the
  // end-of-sequence rule (qw_set_eos)
  bool sampling = false;
  float temperature = 1.f, top_p = 1.f;
  int top_k = 1;
  uint64_t seed = 0;
  int eos = -1;
  int *finished = nullptr;           // [max_batch] 1 once a sequence emitted eos
  // decode-step state (bf16-weight mode): fixed-point residual stream and
  // projection accumulators, LM-head argmax partials
  bool fast_decode = false;
  long long *x_fix = nullptr;        // [max_batch, H]
  long long *x_fix2 = nullptr;       // [max_batch, H] second residual buffer (fused MLP, ping-pong)
  long long *qkv_fix = nullptr;      // [max_batch, nq*hd + 2*nkv*hd]
  long long *gu_fix = nullptr;       // [max_batch, 2I]
  float *arg_v = nullptr;            // [max_batch, ceil(V / 64)]
  int *arg_i = nullptr;
  float *att_m = nullptr, *att_l = nullptr, *att_o = nullptr;   // split-KV partials
  float *norm_ss = nullptr;          // [max_batch, kNormPartsMax] row-norm hand-off sums
  int *sync = nullptr;               // [kSyncCounters] last-arrival counters (zero between kernels)
  void *v_t = nullptr;               // prefill: V of the prompt transposed (f16 mode)
  float *splitk_ws = nullptr;        // prefill split-K slices, sized at creation
  size_t splitk_bytes = 0;
  int batch = 0, pos = 0;
  // decode graph, captured against the staging rows (so caller pointers may
  // change from step to step) for the batch of the last prefill
  bool use_graph = true;
  bool graph_ok = false;
  int graph_batch = 0;
  int graph_variant = -1;
  hipGraphExec_t gexec = nullptr;
  // kernel timing
  int timing_family = -1;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_used, ev_free;
  double timing_ms = 0;
  int64_t timing_n = 0;
  std::vector<void *> allocs;

  KvMap kv() const {
    KvMap k;
    k.table = paged ? block_table : nullptr;
    k.blocks_per_seq = blocks_per_seq;
    k.max_seq = cfg.max_seq;
    return k;
  }

  hipError_t alloc(void **p, size_t bytes) {
    *p = nullptr;
    if (bytes == 0) bytes = 256;
    hipError_t e = hipMalloc(p, bytes);
    if (e == hipSuccess) allocs.push_back(*p);
    return e;
  }
};

namespace {

// Workgroups a decode projection / attention launch aims for (256 CUs).
constexpr int kGemvTargetGroups = 1024;
// With more than two rows every K slice also adds B fixed-point sums per row
// with atomics, so fewer, longer slices pay off.
constexpr int kGemvTargetGroupsBatched = 256;
// split-KV workgroups to aim for (two per CU): at 32 rows x 8k keys 8 splits
// of ~1k keys beat 16 of ~512 (57.3 vs 60.5 us per launch, same box)
constexpr int kAttnTargetGroups = 512;
// Up to this many rows, a projection normalises its own operand (each
// workgroup reads the whole residual rows); above it the residual
// projections hand the norm's operand to the next projection (a norm kernel
// where they cannot).
constexpr int kFusedNormRows = 2;
constexpr bool kHeadNormKernel = true;
#ifndef QW_NORM_HANDOFF
#define QW_NORM_HANDOFF 1
#endif
constexpr bool kNormHandOff = QW_NORM_HANDOFF;
#ifndef QW_TILED_DECODE
#define QW_TILED_DECODE 1
#endif
// more than two rows: projections read unit-tiled weights and operands
constexpr bool kTiledDecode = QW_TILED_DECODE;
#ifndef QW_TILED_PREFILL
#define QW_TILED_PREFILL 1
#endif
// prefill and the LM head over row batches: the MFMA GEMMs read unit-tiled
// weights and operands (A and W stages land as whole 1 KB tiles)
constexpr bool kTiledPrefill = QW_TILED_PREFILL;
// Up to this context length (and two rows), attention and the o projection
// are one kernel in which every workgroup reads its head's whole context;
// past it the split-KV kernel and the o projection (measured: the merged
// kernel wins at 0.5B / 256 keys, the split pair at 1.5B / 513-768 keys).
constexpr int kAttnOMaxCtx = 256;

// Per-step buffers of the fast decode step.  Everything in them is written
// and read within one step; the accumulators are cleared by the step's own
// kernels before they are added into, so their contents between steps do
// not matter.
struct DecodeScratch {
  long long *x_fix = nullptr, *x_fix2 = nullptr;   // [kXReps][B, H] each (two residual buffers)
  long long *qkv_fix = nullptr;                    // [B, nqkv]
  long long *gu_fix = nullptr;                     // [B, 2I]; only the one/two-row path without the fused MLP
  float *arg_v = nullptr;                          // [B, ceil(V / 64)]
  int *arg_i = nullptr;
  float *att_m = nullptr, *att_l = nullptr, *att_o = nullptr;   // [B][nq][16] (+ [hd])
  void *u = nullptr, *o = nullptr, *h = nullptr;   // f16 [B, H], [B, qd], [B, I]
  float *logits = nullptr;                         // [B, V], or NULL (argmax partials only)
  float *norm_ss = nullptr;                        // [B, kNormPartsMax] row-norm hand-off sums
  int *sync = nullptr;                             // [kSyncCounters] last-arrival counters, zero between kernels
};

// Which decode step the next decode call runs: 1 = attention merged with the
// o projection (short context), 2 + S = split-KV attention over S splits,
// then the o projection (S follows the context length, so it grows as the
// sequence does), 0 = the generic (fp32) step.  A captured graph is only
// replayed for the variant it was captured with.
int decode_variant(const qw_model *m) {
  const qw_config &c = m->cfg;
  if (!m->fast_decode) return 0;
  if (m->batch <= kFusedNormRows && m->pos + 1 <= kAttnOMaxCtx && dec_attn_o_supported(c.head_dim, c.hidden))
    return 1;
  return 2 + dec_attn_splits(m->batch, c.n_kv_heads, m->pos + 1, kAttnTargetGroups);
}

// While timing family `fam`, its kernel launches record an event pair at the
// kernel's own start and end (see QW_LAUNCH); the pairs are read back by
// qw_timing_read.
template <class F>
hipError_t timed(qw_model *m, hipStream_t s, Family fam, F &&launch) {
  (void)s;
  if (m->timing_family != fam) return launch();
  std::pair<hipEvent_t, hipEvent_t> ev;
  if (!m->ev_free.empty()) {
    ev = m->ev_free.back();
    m->ev_free.pop_back();
  } else {
    hipError_t e = hipEventCreate(&ev.first);
    if (e == hipSuccess) e = hipEventCreate(&ev.second);
    if (e != hipSuccess) return e;
  }
  launch_timing.start = ev.first;
  launch_timing.stop = ev.second;
  hipError_t e = launch();
  launch_timing = LaunchTiming();
  m->ev_used.push_back(ev);
  return e;
}

// W_tl: the unit-tiled copy of W, with A unit-tiled too (NULL: both
// row-major); h_tiled: a SwiGLU projection writes h unit-tiled
hipError_t gemm(qw_model *m, hipStream_t s, Family fam, const void *A, int M, int K, int lda, const void *W, int N,
                float scale, Epi epi, float *out_f32, void *act_out, int ldo, const QkvRopeArgs *qr = nullptr,
                const void *W_tl = nullptr, bool h_tiled = false) {
  GemmArgs a;
  if (qr) a.qr = *qr;
  if (W_tl) {
    W = W_tl;
    a.tiled = 1;
  }
  a.h_tiled = h_tiled;
  a.A = A;
  a.W = W;
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda = lda;
  a.scale = scale;
  a.epi = epi;
  a.out_f32 = out_f32;
  a.act_out = act_out;
  a.ldo = ldo;
  if (m->f16 && gemm_mfma_supported(a)) {
    const int S = gemm_mfma_splits(M, N, K);
    if (S > 1) {
      // sized in qw_create for every shape a call can reach (splitk_bytes_for)
      if ((size_t)S * M * N * 4 > m->splitk_bytes) return hipErrorInvalidValue;
      a.splits = S;
      a.ws = m->splitk_ws;
    }
    return timed(m, s, fam, [&] { return launch_gemm_mfma(s, a); });
  }
  if (a.tiled || a.h_tiled) return hipErrorInvalidValue;     // tiled operands only on the MFMA kernels
  return timed(m, s, fam, [&] { return launch_gemm_generic(s, m->f16, a); });
}

// A ragged prefill's layout on the device (cu, pcu and the query-tile list
// in rag_meta) and the longest sequence.
struct RaggedPlan {
  RaggedRows rows;
  const int *tiles = nullptr;
  int n_tiles = 0, max_len = 0;
};

// The decoder blocks over T rows (rows_per_seq rows per sequence, the first at
// position pos0, or at pos_dev[b] when pos_dev is given; or the ragged
// sequences of `rag`, each from position 0); x holds the embedded rows on
// entry and the final residual stream on exit.
hipError_t run_layers(qw_model *m, hipStream_t s, int T, int rows_per_seq, int pos0, const int *pos_dev,
                      const RaggedPlan *rag = nullptr) {
  const qw_config &c = m->cfg;
  const int H = c.hidden, I = c.intermediate;
  // Prompt rows from position 0 in f16 mode, when the q/k/v projection runs
  // with K split (short prompts): bias + RoPE + the q and cache writes in its
  // split-K reduction, replacing the separate kernel (1.5B, 512-token prompt:
  // TTFT 5.40 -> 5.20 ms).  Done in the epilogue of an unsplit projection it
  // cost more than the kernel it saves (32 x 8192: 49 + 29 -> 76 + 0 ms per
  // prefill: scattered 2-byte stores, and every load wait also waits for the
  // stores before it).
  GemmArgs probe;
  probe.epi = Epi::QkvRope;
  probe.M = T;
  probe.K = H;
  probe.lda = H;
  probe.N = m->nqkv;
  probe.qr.head_dim = c.head_dim;
  const bool fuse_rope = m->f16 && !pos_dev && pos0 == 0 && gemm_mfma_supported(probe);
  // the GEMM operands u, o and h unit-tiled, with the tiled weight copies,
  // where every producer writes that layout (the prefill attention among them)
  const bool tiled = kTiledPrefill && m->f16 && !pos_dev && pos0 == 0 && attn_prefill_supported(c.head_dim) &&
                     m->L[0].tl_qkv && H % 32 == 0 && H <= kRmsTiledMaxHidden && m->qd % 32 == 0 &&
                     I % 64 == 0;
  auto tl = [&](const void *w) -> const void * { return tiled ? w : nullptr; };
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerBuf &Lw = m->L[l];
    hipError_t e;
    e = timed(m, s, F_RMSNORM,
              [&] { return launch_rmsnorm(s, m->f16, m->x, T, H, H, Lw.in_norm, c.rms_eps, m->u, tiled); });
    if (e != hipSuccess) return e;
    char *kc = (char *)m->k_cache + (int64_t)l * m->cache_layer_elems * m->esz;
    char *vc = (char *)m->v_cache + (int64_t)l * m->cache_layer_elems * m->esz;
    if (fuse_rope) {
      QkvRopeArgs qr;
      qr.bias = Lw.b_qkv;
      qr.rope = m->rope;
      qr.q_out = m->q;
      qr.k_cache = kc;
      qr.v_cache = vc;
      qr.kv = m->kv();
      if (rag) qr.rag = rag->rows;
      qr.rows_per_seq = rows_per_seq;
      qr.n_heads = c.n_heads;
      qr.n_kv_heads = c.n_kv_heads;
      qr.head_dim = c.head_dim;
      e = gemm(m, s, F_GEMM_QKV, m->u, T, H, H, Lw.w_qkv, m->nqkv, Lw.s_qkv, Epi::QkvRope, nullptr, nullptr, 0, &qr,
               tl(Lw.tl_qkv));
      if (e != hipSuccess) return e;
    } else {
    e = gemm(m, s, F_GEMM_QKV, m->u, T, H, H, Lw.w_qkv, m->nqkv, Lw.s_qkv, Epi::StoreF32, m->qkv, nullptr, m->nqkv,
             nullptr, tl(Lw.tl_qkv));
    if (e != hipSuccess) return e;
    RopeCacheArgs ra;
    ra.qkv = m->qkv;
    ra.bias = Lw.b_qkv;
    ra.rope = m->rope;
    ra.q_out = m->q;
    ra.k_cache = kc;
    ra.v_cache = vc;
    ra.kv = m->kv();
    if (rag) ra.rag = rag->rows;
    ra.T = T;
    ra.rows_per_seq = rows_per_seq;
    ra.n_heads = c.n_heads;
    ra.n_kv_heads = c.n_kv_heads;
    ra.head_dim = c.head_dim;
    ra.pos0 = pos0;
    ra.pos0_dev = pos_dev;
    e = timed(m, s, F_ROPE_CACHE, [&] { return launch_rope_cache(s, m->f16, ra); });
    if (e != hipSuccess) return e;
    }
    AttnArgs aa;
    aa.q = m->q;
    aa.k_cache = kc;
    aa.v_cache = vc;
    aa.kv = m->kv();
    aa.tiles = nullptr;
    aa.n_tiles = 0;
    if (rag) {
      aa.rag = rag->rows;
      aa.tiles = rag->tiles;
      aa.n_tiles = rag->n_tiles;
    }
    aa.o = m->o;
    aa.T = T;
    aa.rows_per_seq = rows_per_seq;
    aa.n_heads = c.n_heads;
    aa.n_kv_heads = c.n_kv_heads;
    aa.head_dim = c.head_dim;
    aa.pos0 = pos0;
    aa.pos0_dev = pos_dev;
    aa.softmax_scale = 1.0f / sqrtf((float)c.head_dim);
    aa.v_t = m->v_t;
    aa.o_tiled = tiled;
    if (m->f16 && !pos_dev && pos0 == 0 && attn_prefill_supported(c.head_dim)) {
      const int B = rag ? rag->rows.n : T / rows_per_seq;
      const int max_len = rag ? rag->max_len : rows_per_seq;
      e = timed(m, s, F_ROPE_CACHE, [&] {
        return launch_transpose_v(s, vc, m->kv(), aa.rag, B, c.n_kv_heads, c.head_dim, rows_per_seq, max_len,
                                  m->v_t);
      });
      if (e != hipSuccess) return e;
      e = timed(m, s, F_ATTENTION, [&] { return launch_attention_prefill(s, aa); });
    } else
      e = timed(m, s, F_ATTENTION, [&] { return launch_attention_generic(s, m->f16, aa); });

    if (e != hipSuccess) return e;
    e = gemm(m, s, F_GEMM_O, m->o, T, m->qd, m->qd, Lw.w_o, H, Lw.s_o, Epi::ResidAdd, m->x, nullptr, H, nullptr,
             tl(Lw.tl_o));
    if (e != hipSuccess) return e;
    e = timed(m, s, F_RMSNORM,
              [&] { return launch_rmsnorm(s, m->f16, m->x, T, H, H, Lw.post_norm, c.rms_eps, m->u, tiled); });
    if (e != hipSuccess) return e;
    e = gemm(m, s, F_GEMM_GATE_UP, m->u, T, H, H, Lw.w_gu, 2 * I, Lw.s_gu, Epi::SwiGLU, nullptr, m->h, I, nullptr,
             tl(Lw.tl_gu), tiled);
    if (e != hipSuccess) return e;
    e = gemm(m, s, F_GEMM_DOWN, m->h, T, I, I, Lw.w_down, H, Lw.s_down, Epi::ResidAdd, m->x, nullptr, H, nullptr,
             tl(Lw.tl_down));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Final norm of `rows` residual rows (row r at x + r * stride floats), LM head
// into logits [rows, V], and argmax of `arg_rows` rows of those logits.
hipError_t run_head(qw_model *m, hipStream_t s, const float *x_rows, int rows, int stride, float *logits,
                    const float *arg_logits, int arg_rows, int64_t arg_stride, int32_t *next, int *pos_dev,
                    int pos_add) {
  const qw_config &c = m->cfg;
  // the normed rows unit-tiled for the tiled head copy; not for one row
  // (measured: 1.5B head 0.130 -> 0.148 ms tiled at one row, 0.152 -> 0.145
  // at eight)
  const bool tiled = kTiledPrefill && m->head_tl != nullptr && rows > 1 && c.hidden <= kRmsTiledMaxHidden;
  hipError_t e = timed(m, s, F_RMSNORM, [&] {
    return launch_rmsnorm(s, m->f16, x_rows, rows, stride, c.hidden, m->final_norm, c.rms_eps, m->u, tiled);
  });
  if (e != hipSuccess) return e;
  e = gemm(m, s, F_LM_HEAD, m->u, rows, c.hidden, c.hidden, m->head, c.vocab, m->head_scale, Epi::StoreF32, logits,
           nullptr, c.vocab, nullptr, tiled ? m->head_tl : nullptr);
  if (e != hipSuccess) return e;
  return timed(m, s, F_ARGMAX,
               [&] { return launch_argmax(s, arg_logits, arg_rows, c.vocab, arg_stride, next, pos_dev, pos_add, m->status); });
}

// After the greedy choice of `next` and the position update: the sampled
// choice instead (logits rows of stride `row_stride`), and the end-of-
// sequence rule.
hipError_t choose_next(qw_model *m, hipStream_t s, const float *logits, int64_t row_stride, int B, int32_t *next) {
  int *fin = m->eos >= 0 ? m->finished : nullptr;
  if (m->sampling)
    return launch_sample(s, logits, row_stride, B, m->cfg.vocab, m->temperature, m->top_k, m->top_p, m->seed,
                         m->pos_dev, next, fin, m->eos);
  if (fin) return launch_eos(s, next, fin, m->eos, B);
  return hipSuccess;
}

// Generic decode step (fp32 mode): the prefill kernels on one row per sequence.
hipError_t decode_generic(qw_model *m, hipStream_t s, const int32_t *ids, int32_t *next) {
  const qw_config &c = m->cfg;
  const int B = m->batch;
  hipError_t e = timed(m, s, F_EMBED, [&] {
    return launch_embed(s, m->f16, ids, B, 1, 1, m->emb, m->emb_scale, c.hidden, c.vocab, m->x, m->status);
  });
  if (e != hipSuccess) return e;
  e = run_layers(m, s, B, 1, 0, m->pos_dev);
  if (e != hipSuccess) return e;
  e = run_head(m, s, m->x, B, c.hidden, m->logits, m->logits, B, c.vocab, next, m->pos_dev, 1);
  if (e != hipSuccess) return e;
  return choose_next(m, s, m->logits, c.vocab, B, next);
}

DecGemvArgs dec_args(int *status, const void *W, int M, int N, int K, float scale,
                     int target = kGemvTargetGroups) {
  DecGemvArgs g{};
  g.num_flag = status;
  g.W = W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.scale = scale;
  g.splits = dec_gemv_splits(N, K, M, target);
  return g;
}

// Decode step of the bf16-weight mode (kernels of k_decode.hip): per layer
// [norm] q/k/v projection, attention (bias, RoPE, cache write, split-KV),
// o projection (merging the attention splits), then the MLP; then the LM head
// with per-block argmax and the argmax reduction.  For batches of up to two
// rows the norms are folded into the projection that follows them and the
// MLP is one kernel (norm, gate/up, SwiGLU, down) that reads the residual
// from one buffer and accumulates into the other; for larger batches the
// gate/up projection (SwiGLU in its epilogue) and the down projection run
// separately on one residual buffer, and each residual projection hands the
// next RMSNorm its operand (u without 1/rms, per-row sums of squares).
// Which per-step buffers a fast decode step of B rows uses.
struct DecodeNeeds {
  bool fused_norm, fused_mlp, gu_fix;
};
DecodeNeeds decode_needs(const qw_model *m, int B) {
  DecodeNeeds n;
  n.fused_norm = B <= kFusedNormRows && m->cfg.hidden <= 4096;
  n.fused_mlp = n.fused_norm && m->L[0].w_down_t != nullptr;
  n.gu_fix = n.fused_norm && !n.fused_mlp;
  return n;
}

hipError_t decode_fast(qw_model *m, hipStream_t s, const int32_t *ids, int32_t *next, const DecodeScratch &d) {
  const qw_config &c = m->cfg;
  const int B = m->batch, H = c.hidden, I = c.intermediate, V = c.vocab;
  const DecodeNeeds need = decode_needs(m, B);
  const bool fused_norm = need.fused_norm;
  // one-kernel MLP: reads the residual from xr and accumulates xr + MLP into
  // xo, then the two swap
  const bool fused_mlp = need.fused_mlp;
  // the gate/up sums of the unfused one/two-row MLP (cleared by attention)
  long long *gu_clear = need.gu_fix ? d.gu_fix : nullptr;
  long long *xr = d.x_fix, *xo = d.x_fix2;
  // attention merged with the o projection: the q/k/v sums are still being
  // read in that kernel, so the next projection clears them instead
  const int variant = decode_variant(m);
  const bool attn_o = variant == 1;
  const int S = variant >= 2 ? variant - 2 : 1;
  // the residual is kXReps fixed-point replicas xs apart (value = their sum)
  const int64_t xs = (int64_t)B * H;
  const int64_t n_qkv = (int64_t)B * m->nqkv, n_gu = (int64_t)B * 2 * I;
  // more than two rows: each residual projection hands the next RMSNorm its
  // operand (u without 1/rms, sums of squares per column block), so no norm
  // kernel runs; `parts` sums per row (1 after the embedding)
  const int parts = fused_norm ? 0 : std::min(dec_norm_parts(B, H, m->qd), dec_norm_parts(B, H, I));
  const bool hand = parts > 0 && kNormHandOff;
  // with the hand-off, the projections' weights and f16 operands (u, o, h)
  // are unit-tiled (the producers of u, o and h write that layout)
  const bool tiled = kTiledDecode && hand && m->L[0].tl_qkv != nullptr;
  // (the final norm's operand, read only by the LM head's row-wise staging,
  // keeps the row layout)
  auto hand_out = [&](const float *w, bool row_layout = false) {
    RowNormOut r{};
    if (!hand) return r;
    r.w = w;
    r.u = d.u;
    r.ss = d.norm_ss;
    r.ss_ld = kNormPartsMax;
    r.counters = d.sync;
    r.rep_stride = xs;
    r.tiled = tiled && !row_layout;
    return r;
  };
  // every decode projection reads the unit-tiled weight copy; the operand is
  // tiled too in the batched step with the hand-off
  auto use_tiled = [&](DecGemvArgs &g, const void *w_tl) {
    if (!w_tl) return;
    g.W = w_tl;
    g.w_tiled = 1;
    g.act_tiled = tiled;
  };
  auto hand_in = [&](int n_parts) {
    RowNormIn r{};
    if (!hand) return r;
    r.ss = d.norm_ss;
    r.ss_ld = kNormPartsMax;
    r.parts = n_parts;
    r.dim = (float)H;
    r.eps = c.rms_eps;
    return r;
  };
  hipError_t e = timed(m, s, F_EMBED, [&] {
    // the embedding goes to replica 0; the other replicas and the q/k/v
    // accumulator are cleared (attention clears the gate/up accumulator)
    return launch_dec_embed(s, ids, B, m->emb, m->emb_scale, H, V, d.x_fix, m->status, d.qkv_fix, n_qkv,
                            d.x_fix + xs, (kXReps - 1) * xs, hand_out(m->L[0].in_norm));
  });
  if (e != hipSuccess) return e;
  // operand of a projection that follows an RMSNorm
  auto normed = [&](DecGemvArgs &g, const float *w) {
    g.lda = H;
    if (fused_norm) {
      g.act_mode = 1;
      g.x_fix = xr;
      g.x_rep_stride = xs;
      g.norm_w = w;
      g.eps = c.rms_eps;
    } else {
      g.act_mode = 0;
      g.act = d.u;
    }
  };
  auto norm = [&](const float *w) -> hipError_t {
    if (fused_norm || hand) return hipSuccess;
    return timed(m, s, F_RMSNORM, [&] { return launch_dec_norm(s, xr, xs, B, H, w, c.rms_eps, d.u); });
  };
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerBuf &Lw = m->L[l];
    char *kc = (char *)m->k_cache + (int64_t)l * m->cache_layer_elems * m->esz;
    char *vc = (char *)m->v_cache + (int64_t)l * m->cache_layer_elems * m->esz;
    if ((e = norm(Lw.in_norm)) != hipSuccess) return e;
    const int gemv_target = fused_norm ? kGemvTargetGroups : kGemvTargetGroupsBatched;
    DecGemvArgs g = dec_args(m->status, Lw.w_qkv, B, m->nqkv, H, Lw.s_qkv, gemv_target);
    normed(g, Lw.in_norm);
    g.nin = hand_in(l == 0 ? 1 : parts);
    use_tiled(g, Lw.tl_qkv);
    g.out_fix = d.qkv_fix;
    g.ldo = m->nqkv;
    e = timed(m, s, F_GEMM_QKV, [&] { return launch_dec_gemv(s, g); });
    if (e != hipSuccess) return e;
    if (attn_o) {
      DecAttnOArgs ao{};
      ao.qkv_fix = d.qkv_fix;
      ao.bias = Lw.b_qkv;
      ao.rope = m->rope;
      ao.k_cache = kc;
      ao.v_cache = vc;
      ao.batch = B;
      ao.n_heads = c.n_heads;
      ao.n_kv_heads = c.n_kv_heads;
      ao.head_dim = c.head_dim;
      ao.kv = m->kv();
      ao.pos_dev = m->pos_dev;
      ao.softmax_scale = 1.0f / sqrtf((float)c.head_dim);
      ao.w_o = Lw.w_o;
      ao.w_o_tl = Lw.tl_o;
      ao.o_scale = Lw.s_o;
      ao.H = H;
      ao.x_out = xr;
      ao.clear = fused_mlp ? xo : gu_clear;
      ao.clear_n = fused_mlp ? kXReps * xs : n_gu;
      ao.num_flag = m->status;
      e = timed(m, s, F_ATTN_O, [&] { return launch_dec_attn_o(s, ao); });
      if (e != hipSuccess) return e;
    } else {
      DecAttnArgs da{};
      da.qkv_fix = d.qkv_fix;
      da.bias = Lw.b_qkv;
      da.rope = m->rope;
      da.k_cache = kc;
      da.v_cache = vc;
      da.o = d.o;
      da.part_m = d.att_m;
      da.part_l = d.att_l;
      da.part_o = d.att_o;
      da.splits = S;
      da.head_parallel = B <= kFusedNormRows;      // latency-bound: split the heads over the waves
      da.batch = B;
      da.n_heads = c.n_heads;
      da.n_kv_heads = c.n_kv_heads;
      da.head_dim = c.head_dim;
      da.kv = m->kv();
      da.pos_dev = m->pos_dev;
      da.softmax_scale = 1.0f / sqrtf((float)c.head_dim);
      da.clear = fused_mlp ? xo : gu_clear;
      da.clear_n = fused_mlp ? kXReps * xs : n_gu;
      da.o_tiled = tiled;
      e = timed(m, s, F_ATTENTION, [&] { return launch_dec_attention(s, da); });
      if (e != hipSuccess) return e;
      g = dec_args(m->status, Lw.w_o, B, H, m->qd, Lw.s_o, gemv_target);
      if (S > 1 && !fused_norm) {
        // many rows: merge once, then an f16 operand
        e = timed(m, s, F_ATTN_MERGE, [&] {
          return launch_dec_merge(s, d.att_m, d.att_l, d.att_o, S, B, c.n_heads, c.head_dim, d.o, tiled);
        });
        if (e != hipSuccess) return e;
        g.act_mode = 0;
        g.act = d.o;
      } else if (S > 1) {
        g.act_mode = 3;
        g.part_m = d.att_m;
        g.part_l = d.att_l;
        g.part_o = d.att_o;
        g.attn_splits = S;
        g.n_heads = c.n_heads;
        g.head_dim = c.head_dim;
      } else {
        g.act_mode = 0;
        g.act = d.o;
      }
      g.lda = m->qd;
      g.out_fix = xr;
      g.ldo = H;
      g.clear = d.qkv_fix;
      g.clear_n = n_qkv;
      g.nout = hand_out(Lw.post_norm);
      use_tiled(g, Lw.tl_o);
      e = timed(m, s, F_GEMM_O, [&] { return launch_dec_gemv(s, g); });
      if (e != hipSuccess) return e;
    }
    if (fused_mlp) {
      DecMlpArgs ma{};
      ma.x_in = xr;
      ma.x_out = xo;
      ma.rep_stride = xs;
      ma.norm_w = Lw.post_norm;
      ma.eps = c.rms_eps;
      ma.w_gu = Lw.w_gu;
      ma.gu_scale = Lw.s_gu;
      ma.w_down_t = Lw.w_down_t;
      ma.w_gu_tiled = Lw.tl_gu;
      ma.down_scale = Lw.s_down;
      ma.M = B;
      ma.H = H;
      ma.I = I;
      ma.clear = attn_o ? d.qkv_fix : nullptr;
      ma.clear_n = n_qkv;
      ma.num_flag = m->status;
      e = timed(m, s, F_MLP, [&] { return launch_dec_mlp(s, ma); });
      if (e != hipSuccess) return e;
      std::swap(xr, xo);
      continue;
    }
    if ((e = norm(Lw.post_norm)) != hipSuccess) return e;
    // every workgroup of a norm-fused projection re-reads the residual rows,
    // so fewer, larger K slices pay off when there are many row blocks
    g = dec_args(m->status, Lw.w_gu, B, 2 * I, H, Lw.s_gu, fused_norm ? kGemvTargetGroups / 2 : kGemvTargetGroups);
    normed(g, Lw.post_norm);
    g.role_gate_up = 1;
    g.nin = hand_in(parts);
    use_tiled(g, Lw.tl_gu);
    g.out_fix = d.gu_fix;
    if (!fused_norm) {
      // many rows: full K per workgroup, SwiGLU in the epilogue, f16 h out
      g.splits = 1;
      g.swiglu_out = 1;
      g.h_out = d.h;
      g.ldh = I;
    }
    if (attn_o) {
      g.clear = d.qkv_fix;
      g.clear_n = n_qkv;
    }
    g.ldo = 2 * I;
    e = timed(m, s, F_GEMM_GATE_UP, [&] { return launch_dec_gemv(s, g); });
    if (e != hipSuccess) return e;
    g = dec_args(m->status, Lw.w_down, B, H, I, Lw.s_down, gemv_target);
    if (fused_norm) {
      g.act_mode = 2;
      g.act_fix = d.gu_fix;
      g.lda = 2 * I;
    } else {
      // many rows: h was written by the gate/up epilogue
      g.act_mode = 0;
      g.act = d.h;
      g.lda = I;
    }
    g.out_fix = xr;
    g.ldo = H;
    g.nout = l + 1 < c.n_layers ? hand_out(m->L[l + 1].in_norm) : hand_out(m->final_norm, true);
    use_tiled(g, Lw.tl_down);
    e = timed(m, s, F_GEMM_DOWN, [&] { return launch_dec_gemv(s, g); });
    if (e != hipSuccess) return e;
  }
  // the LM head has thousands of workgroups: the final row is normalised once
  // by a kernel of its own rather than in every workgroup's prologue
  DecGemvArgs g = dec_args(m->status, m->head, B, V, H, m->head_scale);
  if (m->head_tl) {
    g.W = m->head_tl;
    g.w_tiled = 1;
  }
  if (hand) {
    g.act_mode = 0;
    g.act = d.u;
    g.lda = H;
    g.nin = hand_in(parts);
    // the LM head's operand (and its own weights) keep the row layout
  } else if (kHeadNormKernel || !fused_norm) {
    e = timed(m, s, F_RMSNORM, [&] { return launch_dec_norm(s, xr, xs, B, H, m->final_norm, c.rms_eps, d.u); });
    if (e != hipSuccess) return e;
    g.act_mode = 0;
    g.act = d.u;
    g.lda = H;
  } else {
    normed(g, m->final_norm);
  }
  g.ldo = V;
  g.logits_mode = 1;
  g.logits = d.logits;
  g.arg_v = d.arg_v;
  g.arg_i = d.arg_i;
  e = timed(m, s, F_LM_HEAD, [&] { return launch_dec_gemv(s, g); });
  if (e != hipSuccess) return e;
  e = timed(m, s, F_ARGMAX,
            [&] { return launch_dec_end(s, d.arg_v, d.arg_i, (V + 63) / 64, B, next, m->pos_dev); });
  if (e != hipSuccess) return e;
  return choose_next(m, s, d.logits, V, B, next);
}

// The model's own per-step buffers (allocated by qw_create).
DecodeScratch model_scratch(const qw_model *m) {
  DecodeScratch d;
  d.x_fix = m->x_fix;
  d.x_fix2 = m->x_fix2;
  d.qkv_fix = m->qkv_fix;
  d.gu_fix = m->gu_fix;
  d.arg_v = m->arg_v;
  d.arg_i = m->arg_i;
  d.att_m = m->att_m;
  d.att_l = m->att_l;
  d.att_o = m->att_o;
  d.u = m->u;
  d.o = m->o;
  d.h = m->h;
  d.logits = m->logits;
  d.norm_ss = m->norm_ss;
  d.sync = m->sync;
  return d;
}

// One decode step writing next ids to `next` and logits to m->logits.
hipError_t decode_body(qw_model *m, hipStream_t s, const int32_t *ids, int32_t *next) {
  return m->fast_decode ? decode_fast(m, s, ids, next, model_scratch(m)) : decode_generic(m, s, ids, next);
}

// Every block back in the pool.  Blocks are handed out from the highest
// index down, so a sequence's consecutive positions never sit in adjacent
// ascending blocks (any kernel that ignored the table would read wrong keys).
void reset_blocks(qw_model *m) {
  m->free_blocks.resize(m->num_blocks);
  for (int k = 0; k < m->num_blocks; ++k) m->free_blocks[k] = k;
  for (auto &v : m->seq_blocks) v.clear();
}

void drop_graph(qw_model *m) {
  if (m->gexec) (void)hipGraphExecDestroy(m->gexec);
  m->gexec = nullptr;
  m->graph_ok = false;
}

qw_status validate_config(const qw_config *c) {
  if (c->n_layers < 1 || c->hidden < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 ||
      c->intermediate < 1 || c->vocab < 1 || c->max_batch < 1 || c->max_seq < 1)
    return fail(QW_ERR_INVALID_ARG, "qw_create: every size in qw_config must be >= 1");
  if (c->n_heads % c->n_kv_heads != 0)
    return fail(QW_ERR_INVALID_ARG, "qw_create: n_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_heads,
                c->n_kv_heads);
  if (c->head_dim % 2 != 0) return fail(QW_ERR_INVALID_ARG, "qw_create: head_dim must be even (split-half RoPE)");
  if (c->dtype != QW_F32 && c->dtype != QW_BF16 && c->dtype != QW_F16)
    return fail(QW_ERR_INVALID_ARG, "qw_create: unknown dtype");
  if (c->qkv_bias != 1) return fail(QW_ERR_INVALID_ARG, "qw_create: Qwen2 q/k/v projections carry a bias (qkv_bias=1)");
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps)) return fail(QW_ERR_INVALID_ARG, "qw_create: rms_eps must be finite and >= 0");
  if (!(c->rope_theta > 0.f) || !isfinite(c->rope_theta)) return fail(QW_ERR_INVALID_ARG, "qw_create: rope_theta must be finite and > 0");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(QW_ERR_UNSUPPORTED, "qw_create: head_dim %d not built (32, 64, 128)", c->head_dim);
  if (c->hidden % 64 != 0 || c->intermediate % 64 != 0)
    return fail(QW_ERR_UNSUPPORTED, "qw_create: hidden and intermediate must be multiples of 64");
  const int64_t rows = (int64_t)c->max_batch * c->max_seq;
  if (rows > (1LL << 30) || (int64_t)c->n_heads * c->head_dim > (1 << 20) || c->vocab > (1 << 30))
    return fail(QW_ERR_INVALID_ARG, "qw_create: sizes too large");
  return QW_OK;
}

qw_status validate_weights(const qw_config *c, const qw_weights *w) {
  if (!w->embed || !w->final_norm || !w->layers) return fail(QW_ERR_INVALID_ARG, "qw_create: NULL weight pointer (embed, final_norm or layers)");
  if (!c->tie_embeddings && !w->lm_head) return fail(QW_ERR_INVALID_ARG, "qw_create: lm_head is NULL but tie_embeddings is 0");
  for (int l = 0; l < c->n_layers; ++l) {
    const qw_layer_weights &L = w->layers[l];
    const void *p[] = {L.input_norm, L.q_w, L.q_b, L.k_w, L.k_b, L.v_w, L.v_b, L.o_w, L.post_norm, L.gate_w, L.up_w, L.down_w};
    for (const void *q : p)
      if (!q) return fail(QW_ERR_INVALID_ARG, "qw_create: NULL tensor pointer in layer %d", l);
  }
  return QW_OK;
}

// Power-of-two scale 2^k with max|w| * 2^k < 2^15, so that each bf16 value
// times the scale is an fp16 normal (or zero) and converts exactly.
float f16_scale_for(float absmax) {
  if (!(absmax > 0.f) || !isfinite(absmax)) return 1.f;
  int e;
  frexpf(absmax, &e);           // absmax < 2^e
  int k = 15 - e;
  if (k > 60) k = 60;
  if (k < -60) k = -60;
  return ldexpf(1.f, k);
}

// Largest split-K workspace a call can need: the prefill projections (q/k/v,
// o, gate/up, down) and the LM head over up to max_batch * max_seq rows (all
// of them with logits_all), and the generic decode step over max_batch rows.
// Every GEMM has enough tiles for one K slice once M passes 256 * 512 rows,
// so the rows beyond 2^18 need no look.
size_t splitk_bytes_for(const qw_model *m) {
  if (!m->f16) return 0;
  const qw_config &c = m->cfg;
  struct Shape { int N, K; Epi epi; };
  const Shape shapes[] = {{m->nqkv, c.hidden, Epi::StoreF32}, {c.hidden, m->qd, Epi::ResidAdd},
                          {2 * c.intermediate, c.hidden, Epi::SwiGLU}, {c.hidden, c.intermediate, Epi::ResidAdd},
                          {c.vocab, c.hidden, Epi::StoreF32}};
  const int64_t mmax = m->rows_cap < (1 << 18) ? m->rows_cap : (1 << 18);
  size_t most = 0;
  for (const Shape &sh : shapes)
    for (int64_t M = 1; M <= mmax; ++M) {
      GemmArgs a;
      a.M = (int)M;
      a.N = sh.N;
      a.K = sh.K;
      a.lda = sh.K;
      a.epi = sh.epi;
      if (!gemm_mfma_supported(a)) continue;
      const int S = gemm_mfma_splits(a.M, a.N, a.K);
      const size_t need = S > 1 ? (size_t)S * M * sh.N * 4 : 0;
      if (need > most) most = need;
    }
  return most;
}

}  // namespace

static void release_model(qw_model *m);

extern "C" {

const char *qw_last_error(void) { return g_err.c_str(); }

const char *qw_kernel_names(void) { return kFamilyList; }

}  // extern "C"

// qw_create (num_blocks == 0: dense cache) and qw_create_paged.
static qw_status create_model(const qw_config *cfg, const qw_weights *weights, void *hip_stream, int num_blocks,
                              qw_model **out) {
  if (!out) return fail(QW_ERR_INVALID_ARG, "qw_create: out is NULL");
  *out = nullptr;
  if (!cfg || !weights) return fail(QW_ERR_INVALID_ARG, "qw_create: cfg or weights is NULL");
  qw_status st = validate_config(cfg);
  if (st != QW_OK) return st;
  st = validate_weights(cfg, weights);
  if (st != QW_OK) return st;

  qw_model *m = new qw_model();
  const qw_config &c = *cfg;
  m->cfg = c;
  m->f16 = (c.dtype != QW_F32);
  m->esz = m->f16 ? 2 : 4;
  m->qd = c.n_heads * c.head_dim;
  m->kvd = c.n_kv_heads * c.head_dim;
  m->nqkv = m->qd + 2 * m->kvd;
  m->rows_cap = (int64_t)c.max_batch * c.max_seq;
  m->stream = (hipStream_t)hip_stream;
  const int src_kind = c.dtype == QW_BF16 ? kWeightBF16 : c.dtype == QW_F16 ? kWeightF16 : kWeightF32;
  const int H = c.hidden, I = c.intermediate, V = c.vocab;
  auto cleanup_fail = [&](qw_status s) {
    release_model(m);     // keeps the error message
    return s;
  };
#define CREATE_TRY(expr)                                                                          \
  do {                                                                                            \
    hipError_t e_ = (expr);                                                                       \
    if (e_ != hipSuccess)                                                                         \
      return cleanup_fail(fail(e_ == hipErrorOutOfMemory ? QW_ERR_OUT_OF_MEMORY : QW_ERR_HIP,     \
                               "qw_create: %s: %s", #expr, hipGetErrorString(e_)));              \
  } while (0)

  CREATE_TRY(hipStreamCreateWithFlags(&m->cap, hipStreamNonBlocking));
  hipStream_t s = m->stream;
  CREATE_TRY(hipGetDevice(&m->device));
  if (m->device < 0 || m->device >= kMaxDevices)
    return cleanup_fail(fail(QW_ERR_UNSUPPORTED, "qw_create: device ordinal %d beyond %d", m->device, kMaxDevices));
  {
    // the allocation-free decode step's array on this device (once per device)
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[m->device]) {
      void *p = nullptr;
      CREATE_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      g_scratch_dev[m->device] = p;
    }
  }

  // --- per-tensor-group absmax (only needed for the exact f16 scaling)
  // groups: per layer {qkv, o, gu, down}, then embed, then head (if untied)
  const int n_groups = 4 * c.n_layers + 2;
  std::vector<float> scale(n_groups, 1.f);
  if (m->f16) {
    unsigned *amax_dev = nullptr;
    CREATE_TRY(m->alloc((void **)&amax_dev, n_groups * sizeof(unsigned)));
    CREATE_TRY(hipMemsetAsync(amax_dev, 0, n_groups * sizeof(unsigned), s));
    for (int l = 0; l < c.n_layers; ++l) {
      const qw_layer_weights &Lw = weights->layers[l];
      CREATE_TRY(launch_absmax(s, src_kind, Lw.q_w, (int64_t)m->qd * H, amax_dev + 4 * l));
      CREATE_TRY(launch_absmax(s, src_kind, Lw.k_w, (int64_t)m->kvd * H, amax_dev + 4 * l));
      CREATE_TRY(launch_absmax(s, src_kind, Lw.v_w, (int64_t)m->kvd * H, amax_dev + 4 * l));
      CREATE_TRY(launch_absmax(s, src_kind, Lw.o_w, (int64_t)H * m->qd, amax_dev + 4 * l + 1));
      CREATE_TRY(launch_absmax(s, src_kind, Lw.gate_w, (int64_t)I * H, amax_dev + 4 * l + 2));
      CREATE_TRY(launch_absmax(s, src_kind, Lw.up_w, (int64_t)I * H, amax_dev + 4 * l + 2));
      CREATE_TRY(launch_absmax(s, src_kind, Lw.down_w, (int64_t)H * I, amax_dev + 4 * l + 3));
    }
    CREATE_TRY(launch_absmax(s, src_kind, weights->embed, (int64_t)V * H, amax_dev + 4 * c.n_layers));
    if (!c.tie_embeddings)
      CREATE_TRY(launch_absmax(s, src_kind, weights->lm_head, (int64_t)V * H, amax_dev + 4 * c.n_layers + 1));
    std::vector<unsigned> bits(n_groups);
    CREATE_TRY(hipMemcpyAsync(bits.data(), amax_dev, n_groups * sizeof(unsigned), hipMemcpyDeviceToHost, s));
    CREATE_TRY(hipStreamSynchronize(s));
    for (int g = 0; g < n_groups; ++g) {
      float f;
      memcpy(&f, &bits[g], 4);
      if (!isfinite(f))
        return cleanup_fail(fail(QW_ERR_UNSUPPORTED, "qw_create: a weight of %s is inf or NaN",
                                 g < 4 * c.n_layers ? "a decoder layer" : "the embedding or LM head"));
      scale[g] = f16_scale_for(f);
    }
  }

  // --- packed weight copies
  m->L.resize(c.n_layers);
  const bool dst_f16 = m->f16;
  m->fast_decode = m->f16 && c.max_batch <= 32 &&
                   decode_fast_supported(c.head_dim, c.n_heads / c.n_kv_heads, H, m->qd, I);
  // the fused decode MLP (batches of up to two rows) reads W_down transposed
  const bool with_down_t = m->fast_decode && dec_mlp_supported(H, I);
  // the projections read unit-tiled copies (one 1 KB tile per MFMA
  // operand), prefill and decode alike: made where one of them reads them
  const bool with_tiled = m->f16 && H % 32 == 0 && m->qd % 32 == 0 && I % 32 == 0 &&
                          ((kTiledDecode && m->fast_decode) || (kTiledPrefill && H <= kRmsTiledMaxHidden));
  auto tiled_copy = [&](void **dst, const void *W, int N, int K) -> hipError_t {
    hipError_t e = m->alloc(dst, (size_t)(N + kTileRows - 1) / kTileRows * kTileRows * K * 2);
    if (e != hipSuccess) return e;
    return launch_tile_units(s, W, N, K, *dst);
  };
  const size_t es = m->esz;
  for (int l = 0; l < c.n_layers; ++l) {
    const qw_layer_weights &Lw = weights->layers[l];
    LayerBuf &B = m->L[l];
    CREATE_TRY(m->alloc(&B.w_qkv, (size_t)m->nqkv * H * es));
    CREATE_TRY(m->alloc((void **)&B.b_qkv, (size_t)m->nqkv * 4));
    CREATE_TRY(m->alloc(&B.w_o, (size_t)H * m->qd * es));
    CREATE_TRY(m->alloc(&B.w_gu, (size_t)2 * I * H * es));
    CREATE_TRY(m->alloc(&B.w_down, (size_t)H * I * es));
    CREATE_TRY(m->alloc((void **)&B.in_norm, (size_t)H * 4));
    CREATE_TRY(m->alloc((void **)&B.post_norm, (size_t)H * 4));
    const float sq = scale[4 * l], so = scale[4 * l + 1], sg = scale[4 * l + 2], sd = scale[4 * l + 3];
    CREATE_TRY(launch_convert(s, src_kind, Lw.q_w, (int64_t)m->qd * H, dst_f16, B.w_qkv, 0, sq));
    CREATE_TRY(launch_convert(s, src_kind, Lw.k_w, (int64_t)m->kvd * H, dst_f16, B.w_qkv, (int64_t)m->qd * H, sq));
    CREATE_TRY(launch_convert(s, src_kind, Lw.v_w, (int64_t)m->kvd * H, dst_f16, B.w_qkv,
                              (int64_t)(m->qd + m->kvd) * H, sq));

    CREATE_TRY(launch_convert(s, src_kind, Lw.q_b, m->qd, false, B.b_qkv, 0, 1.f));
    CREATE_TRY(launch_convert(s, src_kind, Lw.k_b, m->kvd, false, B.b_qkv, m->qd, 1.f));
    CREATE_TRY(launch_convert(s, src_kind, Lw.v_b, m->kvd, false, B.b_qkv, m->qd + m->kvd, 1.f));
    CREATE_TRY(launch_convert(s, src_kind, Lw.o_w, (int64_t)H * m->qd, dst_f16, B.w_o, 0, so));
    CREATE_TRY(launch_convert_gu(s, src_kind, Lw.gate_w, Lw.up_w, I, H, dst_f16, B.w_gu, sg));
    CREATE_TRY(launch_convert(s, src_kind, Lw.down_w, (int64_t)H * I, dst_f16, B.w_down, 0, sd));
    if (with_down_t) {
      CREATE_TRY(m->alloc(&B.w_down_t, (size_t)I * H * es));
      CREATE_TRY(launch_convert_t(s, src_kind, Lw.down_w, H, I, B.w_down_t, sd));
    }
    if (with_tiled) {
      CREATE_TRY(tiled_copy(&B.tl_qkv, B.w_qkv, m->nqkv, H));
      CREATE_TRY(tiled_copy(&B.tl_o, B.w_o, H, m->qd));
      CREATE_TRY(tiled_copy(&B.tl_gu, B.w_gu, 2 * I, H));
      CREATE_TRY(tiled_copy(&B.tl_down, B.w_down, H, I));
    }
    CREATE_TRY(launch_convert(s, src_kind, Lw.input_norm, H, false, B.in_norm, 0, 1.f));
    CREATE_TRY(launch_convert(s, src_kind, Lw.post_norm, H, false, B.post_norm, 0, 1.f));
    B.s_qkv = 1.f / sq;
    B.s_o = 1.f / so;
    B.s_gu = 1.f / sg;
    B.s_down = 1.f / sd;
  }
  {
    const float se = scale[4 * c.n_layers];
    CREATE_TRY(m->alloc(&m->emb, (size_t)V * H * es));
    CREATE_TRY(launch_convert(s, src_kind, weights->embed, (int64_t)V * H, dst_f16, m->emb, 0, se));
    m->emb_scale = 1.f / se;
    if (c.tie_embeddings) {
      m->head = m->emb;
      m->head_scale = m->emb_scale;
    } else {
      const float sh = scale[4 * c.n_layers + 1];
      CREATE_TRY(m->alloc(&m->head, (size_t)V * H * es));
      CREATE_TRY(launch_convert(s, src_kind, weights->lm_head, (int64_t)V * H, dst_f16, m->head, 0, sh));
      m->head_scale = 1.f / sh;
    }
    if (with_tiled) CREATE_TRY(tiled_copy(&m->head_tl, m->head, V, H));
    CREATE_TRY(m->alloc((void **)&m->final_norm, (size_t)H * 4));
    CREATE_TRY(launch_convert(s, src_kind, weights->final_norm, H, false, m->final_norm, 0, 1.f));
  }

  // --- cache, RoPE table, workspace
  m->pos_host.assign(c.max_batch, 0);
  m->seq_blocks.resize(c.max_batch);
  if (num_blocks > 0) {
    m->paged = true;
    m->num_blocks = num_blocks;
    m->blocks_per_seq = (c.max_seq + kKvBlock - 1) / kKvBlock;
    m->cache_layer_elems = (int64_t)num_blocks * c.n_kv_heads * kKvBlock * c.head_dim;
    const size_t tb = (size_t)c.max_batch * m->blocks_per_seq * 4;
    CREATE_TRY(m->alloc((void **)&m->block_table, tb));
    CREATE_TRY(hipMemsetAsync(m->block_table, 0, tb, s));    // block 0: every stray entry stays in bounds
    reset_blocks(m);
  } else {
    m->cache_layer_elems = (int64_t)c.max_batch * c.n_kv_heads * c.max_seq * c.head_dim;
  }
  const size_t cache_bytes = (size_t)c.n_layers * m->cache_layer_elems * es;
  CREATE_TRY(m->alloc(&m->k_cache, cache_bytes));
  CREATE_TRY(m->alloc(&m->v_cache, cache_bytes));
  CREATE_TRY(hipMemsetAsync(m->k_cache, 0, cache_bytes, s));
  CREATE_TRY(hipMemsetAsync(m->v_cache, 0, cache_bytes, s));
  CREATE_TRY(m->alloc((void **)&m->rope, (size_t)c.max_seq * (c.head_dim / 2) * sizeof(float2)));
  CREATE_TRY(launch_rope_table(s, m->rope, c.max_seq, c.head_dim, (double)c.rope_theta));
  // (whole 16-row blocks: unit-tiled operands are stored in blocks of 16 rows)
  const size_t R = (std::max<size_t>((size_t)m->rows_cap, (size_t)c.max_batch) + 15) / 16 * 16;
  CREATE_TRY(m->alloc((void **)&m->x, R * H * 4));
  CREATE_TRY(m->alloc(&m->u, R * H * es));
  CREATE_TRY(m->alloc((void **)&m->qkv, R * m->nqkv * 4));
  CREATE_TRY(m->alloc(&m->q, R * m->qd * es));
  CREATE_TRY(m->alloc(&m->o, R * m->qd * es));
  CREATE_TRY(m->alloc(&m->h, R * I * es));
  CREATE_TRY(m->alloc((void **)&m->logits, (size_t)c.max_batch * V * 4));
  m->splitk_bytes = splitk_bytes_for(m);
  if (m->splitk_bytes) CREATE_TRY(m->alloc((void **)&m->splitk_ws, m->splitk_bytes));
  if (m->f16)
    CREATE_TRY(m->alloc(&m->v_t, (size_t)c.max_batch * c.n_kv_heads * c.head_dim * ((c.max_seq + 63) / 64 * 64) * 2));
  const size_t pos_bytes = std::max<size_t>(256, (size_t)c.max_batch * 4);
  CREATE_TRY(m->alloc((void **)&m->pos_dev, pos_bytes));
  m->rag_tiles_cap = c.max_batch * ((c.max_seq + attn_prefill_query_tile() - 1) / attn_prefill_query_tile());
  CREATE_TRY(m->alloc((void **)&m->rag_meta, ((size_t)2 * (c.max_batch + 1) + m->rag_tiles_cap) * 4));
  CREATE_TRY(m->alloc((void **)&m->x_last, (size_t)c.max_batch * H * 4));
  CREATE_TRY(m->alloc((void **)&m->status, 256));
  CREATE_TRY(m->alloc((void **)&m->ids_stage, (size_t)c.max_batch * 4));
  if (m->fast_decode) {
    const size_t nb = (size_t)c.max_batch;
    CREATE_TRY(m->alloc((void **)&m->x_fix, kXReps * nb * H * 8));
    CREATE_TRY(m->alloc((void **)&m->x_fix2, kXReps * nb * H * 8));
    CREATE_TRY(m->alloc((void **)&m->qkv_fix, nb * m->nqkv * 8));
    CREATE_TRY(m->alloc((void **)&m->gu_fix, nb * 2 * I * 8));
    CREATE_TRY(m->alloc((void **)&m->arg_v, nb * ((V + 63) / 64) * 4));
    CREATE_TRY(m->alloc((void **)&m->arg_i, nb * ((V + 63) / 64) * 4));
    const size_t ns = nb * c.n_heads * 16;    // at most 16 attention splits
    CREATE_TRY(m->alloc((void **)&m->att_m, ns * 4));
    CREATE_TRY(m->alloc((void **)&m->att_l, ns * 4));
    CREATE_TRY(m->alloc((void **)&m->att_o, ns * c.head_dim * 4));
    CREATE_TRY(m->alloc((void **)&m->norm_ss, nb * kNormPartsMax * 4));
    CREATE_TRY(m->alloc((void **)&m->sync, kSyncCounters * 4));
    CREATE_TRY(hipMemsetAsync(m->sync, 0, kSyncCounters * 4, s));
  }
  CREATE_TRY(m->alloc((void **)&m->next_stage, (size_t)c.max_batch * 4));
  CREATE_TRY(m->alloc((void **)&m->seq_ids, (size_t)c.max_batch * c.max_seq * 4));
  CREATE_TRY(m->alloc((void **)&m->finished, (size_t)c.max_batch * 4));
  CREATE_TRY(hipMemsetAsync(m->finished, 0, (size_t)c.max_batch * 4, s));
  CREATE_TRY(hipMemsetAsync(m->pos_dev, 0, pos_bytes, s));
  CREATE_TRY(hipMemsetAsync(m->status, 0, 256, s));
  CREATE_TRY(hipStreamSynchronize(s));
#undef CREATE_TRY
  *out = m;
  return QW_OK;
}

extern "C" {

qw_status qw_create(const qw_config *cfg, const qw_weights *weights, void *hip_stream, qw_model **out) {
  g_err.clear();
  return create_model(cfg, weights, hip_stream, 0, out);
}

qw_status qw_create_paged(const qw_config *cfg, const qw_weights *weights, int32_t num_blocks, void *hip_stream,
                          qw_model **out) {
  g_err.clear();
  if (out) *out = nullptr;
  if (num_blocks < 1) return fail(QW_ERR_INVALID_ARG, "qw_create_paged: num_blocks must be >= 1");
  if (cfg && (int64_t)num_blocks * cfg->n_kv_heads * kKvBlock * cfg->head_dim > ((int64_t)1 << 40))
    return fail(QW_ERR_INVALID_ARG, "qw_create_paged: %d blocks is beyond any device", num_blocks);
  return create_model(cfg, weights, hip_stream, num_blocks, out);
}

}  // extern "C"

namespace {

int blocks_for(int positions) { return (positions + kKvBlock - 1) / kKvBlock; }

// Paged cache: fail with CACHE_FULL (changing nothing) unless a new batch of
// n sequences holding lens[b] positions each (len_eq when lens is NULL) fits
// the pool.
qw_status check_pool(const qw_model *m, const int *lens, int len_eq, int n, const char *who) {
  if (!m->paged) return QW_OK;
  int64_t need = 0;
  for (int b = 0; b < n; ++b) need += blocks_for(lens ? lens[b] : len_eq);
  if (need > m->num_blocks)
    return fail(QW_ERR_CACHE_FULL, "%s: the sequences need %lld cache blocks of %d positions, the pool holds %d", who,
                (long long)need, kKvBlock, m->num_blocks);
  return QW_OK;
}

// Paged cache: a new batch.  Every block returns to the pool, then sequence b
// takes the blocks of its first lens[b] positions; the table entries go to
// the device in kernel arguments.  The pool was checked (check_pool).
hipError_t assign_blocks(qw_model *m, hipStream_t s, const int *lens, int len_eq, int n) {
  if (!m->paged) return hipSuccess;
  reset_blocks(m);
  std::vector<int> idx, val;
  for (int b = 0; b < n; ++b) {
    const int nb = blocks_for(lens ? lens[b] : len_eq);
    for (int p = 0; p < nb; ++p) {
      const int blk = m->free_blocks.back();
      m->free_blocks.pop_back();
      m->seq_blocks[b].push_back(blk);
      idx.push_back(b * m->blocks_per_seq + p);
      val.push_back(blk);
    }
  }
  return launch_put_ints(s, m->block_table, idx.data(), val.data(), (int)idx.size());
}

// Paged cache, before a decode step: the block of every sequence whose new
// token starts one.  CACHE_FULL (changing nothing) when the pool has too few.
qw_status reserve_step_blocks(qw_model *m, hipStream_t s, const char *who) {
  if (!m->paged) return QW_OK;
  std::vector<int> need;
  for (int b = 0; b < m->batch; ++b)
    if (m->pos_host[b] / kKvBlock >= (int)m->seq_blocks[b].size()) need.push_back(b);
  if (need.empty()) return QW_OK;
  if ((int)need.size() > (int)m->free_blocks.size())
    return fail(QW_ERR_CACHE_FULL, "%s: %d sequences start a new cache block, %d blocks are free", who,
                (int)need.size(), (int)m->free_blocks.size());
  std::vector<int> idx, val;
  for (int b : need) {
    const int blk = m->free_blocks.back();
    m->free_blocks.pop_back();
    idx.push_back(b * m->blocks_per_seq + (int)m->seq_blocks[b].size());
    val.push_back(blk);
    m->seq_blocks[b].push_back(blk);
  }
  const hipError_t e = launch_put_ints(s, m->block_table, idx.data(), val.data(), (int)idx.size());
  if (e != hipSuccess) return fail(QW_ERR_HIP, "%s: block table update: %s", who, hipGetErrorString(e));
  return QW_OK;
}

// Host positions after a prefill of n sequences (lens[b], or len_eq each).
void set_positions(qw_model *m, const int *lens, int len_eq, int n) {
  int mx = 0;
  for (int b = 0; b < m->cfg.max_batch; ++b) {
    m->pos_host[b] = b < n ? (lens ? lens[b] : len_eq) : 0;
    mx = std::max(mx, m->pos_host[b]);
  }
  m->pos = mx;
}

// Host positions after a decode step: every sequence of the batch holds one more.
void advance_positions(qw_model *m) {
  for (int b = 0; b < m->batch; ++b) m->pos_host[b] += 1;
  m->pos += 1;
}

// The enqueue of a prefill whose arguments are valid: `batch` sequences of
// `prompt_len` ids, sequence b's at ids + b * ids_stride.
hipError_t prefill_enqueue(qw_model *m, const int32_t *ids, int64_t ids_stride, int batch, int prompt_len,
                           float *logits, int logits_all, int32_t *next_ids, bool new_sequences = true) {
  const qw_config &c = m->cfg;
  hipStream_t s = m->stream;
  const int T = batch * prompt_len, H = c.hidden, V = c.vocab;
  hipError_t e = assign_blocks(m, s, nullptr, prompt_len, batch);
  if (e != hipSuccess) return e;
  e = timed(m, s, F_EMBED, [&] {
    return launch_embed(s, m->f16, ids, T, prompt_len, ids_stride, m->emb, m->emb_scale, H, V, m->x, m->status);
  });
  if (e != hipSuccess) return e;
  if ((e = run_layers(m, s, T, prompt_len, 0, nullptr)) != hipSuccess) return e;
  const float *last;                  // each sequence's last-row logits, rows `stride` apart
  int64_t stride;
  if (logits_all) {
    last = logits + (int64_t)(prompt_len - 1) * V;
    stride = (int64_t)prompt_len * V;
    e = run_head(m, s, m->x, T, H, logits, last, batch, stride, next_ids, nullptr, 0);
  } else {
    float *lg = logits ? logits : m->logits;
    last = lg;
    stride = V;
    e = run_head(m, s, m->x + (int64_t)(prompt_len - 1) * H, batch, prompt_len * H, lg, lg, batch, V, next_ids,
                 nullptr, 0);
  }
  if (e != hipSuccess) return e;
  if ((e = launch_fill_int(s, m->pos_dev, prompt_len, batch)) != hipSuccess) return e;
  if (new_sequences && m->eos >= 0 && (e = launch_fill_int(s, m->finished, 0, batch)) != hipSuccess) return e;
  return choose_next(m, s, last, stride, batch, next_ids);
}

// The enqueue of a ragged prefill whose arguments are valid (lens: host).
hipError_t prefill_ragged_enqueue(qw_model *m, const int32_t *ids, const int32_t *lens, int n, float *logits,
                                  int32_t *next_ids) {
  const qw_config &c = m->cfg;
  hipStream_t s = m->stream;
  const int H = c.hidden, V = c.vocab;
  hipError_t e = assign_blocks(m, s, lens, 0, n);
  if (e != hipSuccess) return e;
  // device layout: cu [n + 1], pcu [n + 1] (after max_batch + 1 entries),
  // then the query-tile list, (sequence << 16) | tile, in the order below
  const int off_pcu = c.max_batch + 1, off_tiles = 2 * (c.max_batch + 1);
  std::vector<int> idx, val;
  const int BQ = attn_prefill_query_tile();
  int T = 0, PT = 0, max_len = 0, max_qt = 0;
  for (int b = 0; b <= n; ++b) {
    idx.push_back(b);
    val.push_back(T);
    idx.push_back(off_pcu + b);
    val.push_back(PT);
    if (b < n) {
      T += lens[b];
      PT += blocks_for(lens[b]) * kKvBlock;
      max_len = std::max(max_len, lens[b]);
      max_qt = std::max(max_qt, (lens[b] + BQ - 1) / BQ);
    }
  }
  // The attention kernel deals work item w = tile * nq + head to XCD
  // w / ceil(n_tiles * nq / 8) (workgroups go round-robin over the 8 XCDs,
  // and each XCD walks its range in order).  Tiles are placed heaviest first
  // (cost ~ qt + 1 key blocks) on the XCD with the least work so far that
  // still has room, so the XCDs end together and each starts with its
  // heaviest tiles.
  std::vector<int> order;
  for (int qt = max_qt - 1; qt >= 0; --qt)
    for (int b = 0; b < n; ++b)
      if ((lens[b] + BQ - 1) / BQ > qt) order.push_back((b << 16) | qt);
  const int n_tiles = (int)order.size();
  const int64_t per_x = ((int64_t)n_tiles * c.n_heads + 7) / 8;
  std::vector<std::vector<int>> slots(8);             // tile positions of each XCD, in order
  for (int t = 0; t < n_tiles; ++t) slots[std::min<int64_t>(7, (int64_t)t * c.n_heads / per_x)].push_back(t);
  std::vector<int64_t> load(8, 0);
  std::vector<size_t> used(8, 0);
  std::vector<int> placed(n_tiles);
  for (int it : order) {
    int best = -1;
    for (int x = 0; x < 8; ++x)
      if (used[x] < slots[x].size() && (best < 0 || load[x] < load[best])) best = x;
    placed[slots[best][used[best]++]] = it;
    load[best] += (it & 0xffff) + 1;
  }
  for (int t = 0; t < n_tiles; ++t) {
    idx.push_back(off_tiles + t);
    val.push_back(placed[t]);
  }
  if ((e = launch_put_ints(s, m->rag_meta, idx.data(), val.data(), (int)idx.size())) != hipSuccess) return e;
  RaggedPlan plan;
  plan.rows.cu = m->rag_meta;
  plan.rows.pcu = m->rag_meta + off_pcu;
  plan.rows.n = n;
  plan.tiles = m->rag_meta + off_tiles;
  plan.n_tiles = n_tiles;
  plan.max_len = max_len;
  e = timed(m, s, F_EMBED, [&] {
    return launch_embed(s, m->f16, ids, T, T, T, m->emb, m->emb_scale, H, V, m->x, m->status);
  });
  if (e != hipSuccess) return e;
  if ((e = run_layers(m, s, T, T, 0, nullptr, &plan)) != hipSuccess) return e;
  // the last row of each sequence
  if ((e = launch_gather_last_rows(s, m->x_last, m->x, plan.rows.cu, n, H)) != hipSuccess) return e;
  float *lg = logits ? logits : m->logits;
  if ((e = run_head(m, s, m->x_last, n, H, lg, lg, n, V, next_ids, nullptr, 0)) != hipSuccess) return e;
  std::vector<int> pidx(n), pval(n);
  for (int b = 0; b < n; ++b) {
    pidx[b] = b;
    pval[b] = lens[b];
  }
  if ((e = launch_put_ints(s, m->pos_dev, pidx.data(), pval.data(), n)) != hipSuccess) return e;
  if (m->eos >= 0 && (e = launch_fill_int(s, m->finished, 0, n)) != hipSuccess) return e;
  return choose_next(m, s, lg, V, n, next_ids);
}

}  // namespace

extern "C" {

qw_status qw_prefill(qw_model *m, const int32_t *ids, int32_t batch, int32_t prompt_len, float *logits,
                     int32_t logits_all, int32_t *next_ids) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_prefill: model is NULL");
  if (!ids || !next_ids) return fail(QW_ERR_INVALID_ARG, "qw_prefill: ids and next_ids must be non-NULL");
  const qw_config &c = m->cfg;
  if (batch < 1 || batch > c.max_batch)
    return fail(QW_ERR_INVALID_ARG, "qw_prefill: batch %d outside [1, max_batch=%d]", batch, c.max_batch);
  if (prompt_len < 1) return fail(QW_ERR_INVALID_ARG, "qw_prefill: prompt_len must be >= 1");
  if (prompt_len > c.max_seq)
    return fail(QW_ERR_CACHE_FULL, "qw_prefill: prompt_len %d exceeds max_seq %d", prompt_len, c.max_seq);
  if (logits_all && !logits) return fail(QW_ERR_INVALID_ARG, "qw_prefill: logits_all needs a logits buffer");
  qw_status st = check_pool(m, nullptr, prompt_len, batch, "qw_prefill");
  if (st != QW_OK) return st;
  m->batch = 0;          // invalid until the enqueue succeeds
  HIP_TRY(prefill_enqueue(m, ids, prompt_len, batch, prompt_len, logits, logits_all, next_ids));
  m->batch = batch;
  set_positions(m, nullptr, prompt_len, batch);
  return QW_OK;
}

qw_status qw_prefill_ragged(qw_model *m, const int32_t *ids, const int32_t *lens, int32_t n_seqs, float *logits,
                            int32_t *next_ids) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_prefill_ragged: model is NULL");
  if (!ids || !lens || !next_ids)
    return fail(QW_ERR_INVALID_ARG, "qw_prefill_ragged: ids, lens and next_ids must be non-NULL");
  const qw_config &c = m->cfg;
  if (n_seqs < 1 || n_seqs > c.max_batch)
    return fail(QW_ERR_INVALID_ARG, "qw_prefill_ragged: n_seqs %d outside [1, max_batch=%d]", n_seqs, c.max_batch);
  if (n_seqs >= (1 << 15))
    return fail(QW_ERR_INVALID_ARG, "qw_prefill_ragged: n_seqs %d beyond the tile list's 15 bits", n_seqs);
  for (int b = 0; b < n_seqs; ++b) {
    if (lens[b] < 1) return fail(QW_ERR_INVALID_ARG, "qw_prefill_ragged: lens[%d] = %d (must be >= 1)", b, lens[b]);
    if (lens[b] > c.max_seq)
      return fail(QW_ERR_CACHE_FULL, "qw_prefill_ragged: lens[%d] = %d exceeds max_seq %d", b, lens[b], c.max_seq);
  }
  qw_status st = check_pool(m, lens, 0, n_seqs, "qw_prefill_ragged");
  if (st != QW_OK) return st;
  m->batch = 0;          // invalid until the enqueue succeeds
  HIP_TRY(prefill_ragged_enqueue(m, ids, lens, n_seqs, logits, next_ids));
  m->batch = n_seqs;
  set_positions(m, lens, 0, n_seqs);
  return QW_OK;
}

qw_status qw_get_positions(const qw_model *m, int32_t *pos, int32_t n) {
  g_err.clear();
  if (!m || !pos) return fail(QW_ERR_INVALID_ARG, "qw_get_positions: NULL argument");
  if (n < 0 || n > m->cfg.max_batch)
    return fail(QW_ERR_INVALID_ARG, "qw_get_positions: n %d outside [0, max_batch=%d]", n, m->cfg.max_batch);
  for (int b = 0; b < n; ++b) pos[b] = b < m->batch ? m->pos_host[b] : 0;
  return QW_OK;
}

qw_status qw_kv_blocks(const qw_model *m, int32_t *free_blocks, int32_t *total_blocks) {
  g_err.clear();
  if (!m || !free_blocks || !total_blocks) return fail(QW_ERR_INVALID_ARG, "qw_kv_blocks: NULL argument");
  *total_blocks = m->paged ? m->num_blocks : 0;
  *free_blocks = m->paged ? (int32_t)m->free_blocks.size() : 0;
  return QW_OK;
}

qw_status qw_decode_step(qw_model *m, const int32_t *ids, float *logits, int32_t *next_ids) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_decode_step: model is NULL");
  if (!ids || !next_ids) return fail(QW_ERR_INVALID_ARG, "qw_decode_step: ids and next_ids must be non-NULL");
  if (m->batch == 0) return fail(QW_ERR_BAD_STATE, "qw_decode_step: no prefill has run");
  if (m->pos >= m->cfg.max_seq)
    return fail(QW_ERR_CACHE_FULL, "qw_decode_step: cache holds max_seq=%d positions", m->cfg.max_seq);
  hipStream_t s = m->stream;
  qw_status st = reserve_step_blocks(m, s, "qw_decode_step");
  if (st != QW_OK) return st;
  const bool graph = m->use_graph && m->timing_family < 0;
  if (!graph) {
    HIP_TRY(decode_body(m, s, ids, m->next_stage));
  } else {
    const int variant = decode_variant(m);
    if (!m->graph_ok || m->graph_batch != m->batch || m->graph_variant != variant) {
      drop_graph(m);
      hipGraph_t g = nullptr;
      HIP_TRY(hipStreamBeginCapture(m->cap, hipStreamCaptureModeThreadLocal));
      hipError_t e = decode_body(m, m->cap, m->ids_stage, m->next_stage);
      hipError_t e2 = hipStreamEndCapture(m->cap, &g);
      if (e != hipSuccess || e2 != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return fail(QW_ERR_HIP, "qw_decode_step: graph capture failed: %s",
                    hipGetErrorString(e != hipSuccess ? e : e2));
      }
      e = hipGraphInstantiate(&m->gexec, g, nullptr, nullptr, 0);
      (void)hipGraphDestroy(g);
      if (e != hipSuccess) {
        m->gexec = nullptr;
        return fail(QW_ERR_HIP, "qw_decode_step: graph instantiate failed: %s", hipGetErrorString(e));
      }
      m->graph_batch = m->batch;
      m->graph_variant = variant;
      m->graph_ok = true;
    }
    HIP_TRY(launch_copy_i32(s, m->ids_stage, ids, m->batch));
    HIP_TRY(hipGraphLaunch(m->gexec, s));
  }
  HIP_TRY(launch_stage_out(s, next_ids, m->next_stage, m->batch, logits, m->logits, (int64_t)m->batch * m->cfg.vocab));
  advance_positions(m);
  return QW_OK;
}

qw_status qw_decode_step_noalloc(qw_model *m, const int32_t *ids, float *logits, int32_t *next_ids) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_decode_step_noalloc: model is NULL");
  if (!ids || !next_ids) return fail(QW_ERR_INVALID_ARG, "qw_decode_step_noalloc: ids and next_ids must be non-NULL");
  if (m->batch == 0) return fail(QW_ERR_BAD_STATE, "qw_decode_step_noalloc: no prefill has run");
  if (m->pos >= m->cfg.max_seq)
    return fail(QW_ERR_CACHE_FULL, "qw_decode_step_noalloc: cache holds max_seq=%d positions", m->cfg.max_seq);
  if (!m->fast_decode)
    return fail(QW_ERR_UNSUPPORTED, "qw_decode_step_noalloc: covers the bf16 decode step of up to 32 rows and GQA "
                                    "groups of up to 8 (this model takes the generic step)");
  if (m->sampling && !logits)
    return fail(QW_ERR_INVALID_ARG, "qw_decode_step_noalloc: sampling reads the logits: pass a logits buffer");
  const qw_config &c = m->cfg;
  const int64_t B = m->batch, H = c.hidden, I = c.intermediate, V = c.vocab;
  const int64_t B16 = (B + 15) / 16 * 16;
  const DecodeNeeds need = decode_needs(m, (int)B);
  // carve the step's buffers out of this device's array, 256-byte aligned;
  // the last-arrival counters always sit at its start (zero at load, and
  // every kernel that counts leaves them at zero)
  const int64_t sizes[] = {
      kSyncCounters * 4,                                 // sync
      kXReps * B * H * 8, kXReps * B * H * 8,             // x_fix, x_fix2
      B * m->nqkv * 8,                                   // qkv_fix
      need.gu_fix ? B * 2 * I * 8 : 0,                   // gu_fix
      B * ((V + 63) / 64) * 4, B * ((V + 63) / 64) * 4,   // arg_v, arg_i
      B * c.n_heads * 16 * 4, B * c.n_heads * 16 * 4,     // att_m, att_l (at most 16 splits)
      B * c.n_heads * 16 * c.head_dim * 4,               // att_o
      B16 * H * 2, B16 * m->qd * 2, B16 * I * 2,         // u, o, h (f16; unit-tiled in blocks of 16 rows)
      B * kNormPartsMax * 4,                             // norm_ss
  };
  constexpr int kParts = sizeof(sizes) / sizeof(sizes[0]);
  int64_t off[kParts], total = 0;
  for (int k = 0; k < kParts; ++k) {
    off[k] = total;
    total += (sizes[k] + 255) / 256 * 256;
  }
  if (total > (int64_t)kNoAllocScratchBytes)
    return fail(QW_ERR_UNSUPPORTED, "qw_decode_step_noalloc: a step of %d rows at these shapes needs %lld bytes of "
                "scratch, more than the %zu of the static array", m->batch, (long long)total, kNoAllocScratchBytes);
  char *base = (char *)g_scratch_dev[m->device];
  if (!base) return fail(QW_ERR_BAD_STATE, "qw_decode_step_noalloc: no scratch address for device %d", m->device);
  int dev_now = -1;
  HIP_TRY(hipGetDevice(&dev_now));
  if (dev_now != m->device)
    return fail(QW_ERR_BAD_STATE, "qw_decode_step_noalloc: the model lives on device %d, device %d is current",
                m->device, dev_now);
  qw_status st = reserve_step_blocks(m, m->stream, "qw_decode_step_noalloc");
  if (st != QW_OK) return st;
  DecodeScratch d;
  d.sync = (int *)(base + off[0]);
  d.x_fix = (long long *)(base + off[1]);
  d.x_fix2 = (long long *)(base + off[2]);
  d.qkv_fix = (long long *)(base + off[3]);
  d.gu_fix = need.gu_fix ? (long long *)(base + off[4]) : nullptr;
  d.arg_v = (float *)(base + off[5]);
  d.arg_i = (int *)(base + off[6]);
  d.att_m = (float *)(base + off[7]);
  d.att_l = (float *)(base + off[8]);
  d.att_o = (float *)(base + off[9]);
  d.u = base + off[10];
  d.o = base + off[11];
  d.h = base + off[12];
  d.norm_ss = (float *)(base + off[13]);
  d.logits = logits;                 // the caller's buffer, or none
  // launched one by one on the model's stream (nothing captured or
  // instantiated); kernel timing stays off (it would create events)
  const int fam = m->timing_family;
  m->timing_family = -1;
  hipError_t e = decode_fast(m, m->stream, ids, next_ids, d);
  m->timing_family = fam;
  HIP_TRY(e);
  advance_positions(m);
  return QW_OK;
}

qw_status qw_generate(qw_model *m, const int32_t *ids, int32_t batch, int32_t prompt_len, int32_t steps,
                      int32_t use_cache, int32_t *out_ids, float *logits) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_generate: model is NULL");
  if (!ids || !out_ids) return fail(QW_ERR_INVALID_ARG, "qw_generate: ids and out_ids must be non-NULL");
  const qw_config &c = m->cfg;
  if (batch < 1 || batch > c.max_batch)
    return fail(QW_ERR_INVALID_ARG, "qw_generate: batch %d outside [1, max_batch=%d]", batch, c.max_batch);
  if (prompt_len < 1 || steps < 0) return fail(QW_ERR_INVALID_ARG, "qw_generate: prompt_len >= 1 and steps >= 0");
  if ((int64_t)prompt_len + steps > c.max_seq)
    return fail(QW_ERR_CACHE_FULL, "qw_generate: prompt_len %d + steps %d exceeds max_seq %d", prompt_len, steps,
                c.max_seq);
  qw_status st0 = check_pool(m, nullptr, prompt_len + steps, batch, "qw_generate");
  if (st0 != QW_OK) return st0;
  hipStream_t s = m->stream;
  const int V = c.vocab;
  const int64_t cols = (int64_t)steps + 1;
  // step k's logits are rows b * cols + k of `logits`; its token column k of out_ids
  auto put_logits = [&](int k) -> hipError_t {
    if (!logits) return hipSuccess;
    return launch_copy_rows(s, logits + (int64_t)k * V, cols * V, m->logits, V, batch, V);
  };
  m->batch = 0;
  if (use_cache) {
    HIP_TRY(prefill_enqueue(m, ids, prompt_len, batch, prompt_len, logits ? m->logits : nullptr, 0, m->next_stage));
    m->batch = batch;
    set_positions(m, nullptr, prompt_len, batch);
    HIP_TRY(put_logits(0));
    HIP_TRY(launch_put_column(s, out_ids, cols, 0, nullptr, 0, 0, m->next_stage, batch));
    for (int k = 1; k <= steps; ++k) {
      // the step reads the staging row in place (ids may alias next ids)
      qw_status st = qw_decode_step(m, m->next_stage, logits ? m->logits : nullptr, m->next_stage);
      if (st != QW_OK) return st;
      HIP_TRY(put_logits(k));
      HIP_TRY(launch_put_column(s, out_ids, cols, k, nullptr, 0, 0, m->next_stage, batch));
    }
    return QW_OK;
  }
  // no cache reuse: step k runs a prefill over the prompt and the k tokens
  // generated so far, kept in seq_ids (row stride max_seq)
  const int64_t ss = c.max_seq;
  HIP_TRY(launch_copy_rows(s, m->seq_ids, ss, ids, prompt_len, batch, prompt_len));
  for (int k = 0; k <= steps; ++k) {
    const int L = prompt_len + k;
    HIP_TRY(prefill_enqueue(m, m->seq_ids, ss, batch, L, logits ? m->logits : nullptr, 0, m->next_stage, k == 0));
    HIP_TRY(put_logits(k));
    HIP_TRY(launch_put_column(s, out_ids, cols, k, k < steps ? m->seq_ids : nullptr, ss, L, m->next_stage, batch));
  }
  m->batch = batch;
  set_positions(m, nullptr, prompt_len + steps, batch);
  return QW_OK;
}

qw_status qw_destroy(qw_model *m) {
  g_err.clear();
  release_model(m);
  return QW_OK;
}

}  // extern "C"

// Frees everything a handle owns (also for a half-built handle); leaves the
// thread's last error as it is.
static void release_model(qw_model *m) {
  if (!m) return;
  (void)hipStreamSynchronize(m->stream);
  drop_graph(m);
  for (auto &e : m->ev_used) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  for (auto &e : m->ev_free) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  for (void *p : m->allocs) (void)hipFree(p);
  if (m->cap) (void)hipStreamDestroy(m->cap);
  delete m;
}

extern "C" {

qw_status qw_get_state(const qw_model *m, int32_t *batch, int32_t *pos) {
  g_err.clear();
  if (!m || !batch || !pos) return fail(QW_ERR_INVALID_ARG, "qw_get_state: NULL argument");
  *batch = m->batch;
  *pos = m->batch ? m->pos : 0;
  return QW_OK;
}

// Reads the status word after the stream is idle, clears the bits in `mask`
// and returns those of them that were set.
static qw_status read_status(qw_model *m, int mask, int *bits) {
  HIP_TRY(hipStreamSynchronize(m->stream));
  int word = 0;
  HIP_TRY(hipMemcpy(&word, m->status, sizeof(int), hipMemcpyDeviceToHost));
  *bits = word & mask;
  if (*bits) {
    word &= ~mask;
    HIP_TRY(hipMemcpy(m->status, &word, sizeof(int), hipMemcpyHostToDevice));
  }
  return QW_OK;
}

qw_status qw_check_ids(qw_model *m) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_check_ids: model is NULL");
  int bits = 0;
  qw_status st = read_status(m, kFlagBadId, &bits);
  if (st != QW_OK) return st;
  if (bits) return fail(QW_ERR_INVALID_ARG, "a token id outside [0, %d) was passed; it was read as id 0", m->cfg.vocab);
  return QW_OK;
}

qw_status qw_check_numerics(qw_model *m) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_check_numerics: model is NULL");
  int bits = 0;
  qw_status st = read_status(m, kFlagNonFinite | kFlagFixRange, &bits);
  if (st != QW_OK) return st;
  if (bits)
    return fail(QW_ERR_NUMERICS, "since the last check:%s%s", (bits & kFlagNonFinite) ? " a logit was inf or NaN;" : "",
                (bits & kFlagFixRange) ? " a decode residual or projection addend exceeded 2^23 in magnitude;" : "");
  return QW_OK;
}

qw_status qw_set_sampling(qw_model *m, float temperature, int32_t top_k, float top_p, uint64_t seed) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_set_sampling: model is NULL");
  if (top_k == 0) {
    m->sampling = false;
  } else {
    if (!(temperature > 0.f) || !isfinite(temperature) || top_k < 1 || top_k > 1024 || !(top_p > 0.f) ||
        !(top_p <= 1.f))
      return fail(QW_ERR_INVALID_ARG, "qw_set_sampling: need temperature > 0, 1 <= top_k <= 1024 (0: greedy), "
                                      "0 < top_p <= 1");
    m->sampling = true;
    m->temperature = temperature;
    m->top_k = top_k;
    m->top_p = top_p;
    m->seed = seed;
  }
  drop_graph(m);
  return QW_OK;
}

qw_status qw_set_eos(qw_model *m, int32_t eos_id) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_set_eos: model is NULL");
  if (eos_id < -1 || eos_id >= m->cfg.vocab)
    return fail(QW_ERR_INVALID_ARG, "qw_set_eos: eos_id %d outside [-1, %d)", eos_id, m->cfg.vocab);
  m->eos = eos_id;
  drop_graph(m);
  return QW_OK;
}

qw_status qw_get_finished(qw_model *m, int32_t *finished, int32_t n) {
  g_err.clear();
  if (!m || !finished || n < 0 || n > m->cfg.max_batch)
    return fail(QW_ERR_INVALID_ARG, "qw_get_finished: model, host buffer and 0 <= n <= max_batch needed");
  HIP_TRY(hipStreamSynchronize(m->stream));
  if (m->eos < 0) {
    memset(finished, 0, (size_t)n * 4);
    return QW_OK;
  }
  HIP_TRY(hipMemcpy(finished, m->finished, (size_t)n * 4, hipMemcpyDeviceToHost));
  return QW_OK;
}

qw_status qw_set_graph(qw_model *m, int32_t enable) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_set_graph: model is NULL");
  m->use_graph = enable != 0;
  if (!m->use_graph) drop_graph(m);
  return QW_OK;
}

qw_status qw_timing_enable(qw_model *m, const char *name) {
  g_err.clear();
  if (!m) return fail(QW_ERR_INVALID_ARG, "qw_timing_enable: model is NULL");
  if (!name || !*name) {
    m->timing_family = -1;
    return QW_OK;
  }
  for (int f = 0; f < F_COUNT; ++f)
    if (strcmp(name, kFamilyNames[f]) == 0) {
      m->timing_family = f;
      return QW_OK;
    }
  return fail(QW_ERR_INVALID_ARG, "qw_timing_enable: unknown kernel family '%s' (have: %s)", name, kFamilyList);
}

qw_status qw_timing_read(qw_model *m, double *total_ms, int64_t *launches, int32_t reset) {
  g_err.clear();
  if (!m || !total_ms || !launches) return fail(QW_ERR_INVALID_ARG, "qw_timing_read: NULL argument");
  HIP_TRY(hipStreamSynchronize(m->stream));
  for (auto &e : m->ev_used) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, e.first, e.second));
    m->timing_ms += ms;
    m->timing_n += 1;
    m->ev_free.push_back(e);
  }
  m->ev_used.clear();
  *total_ms = m->timing_ms;
  *launches = m->timing_n;
  if (reset) {
    m->timing_ms = 0;
    m->timing_n = 0;
  }
  return QW_OK;
}

}  // extern "C"
