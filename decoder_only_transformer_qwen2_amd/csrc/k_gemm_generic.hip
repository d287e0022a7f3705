// Generic tiled GEMM  C[M, N] = A[M, K] . W[N, K]^T  on the vector ALUs, with
// fp32 accumulation and the three epilogues of the decoder block:
//   StoreF32  q/k/v projections (bias and RoPE follow in rope_cache) and logits
//   ResidAdd  o_proj and down_proj added into the fp32 residual stream
//             ("LLM Speedrun: Architecture", section "Gradients be vanishing
//             or activations exploding": residual connections)
//   SwiGLU    gate/up projection followed by silu(gate) * up ("But how does it
//             remember things?"; "augur": Qwen MLP)
// This is the fp32 path (and a fallback for shapes the MFMA kernels do not
// take); weights are the library's packed copies in the compute type.
#include "qw_internal.h"

namespace qw {

namespace {
constexpr int TM = 64, TN = 64, TK = 32;

template <typename T>
__global__ void __launch_bounds__(256) gemm_generic_kernel(GemmArgs a) {
  __shared__ float As[TK][TM + 1];
  __shared__ float Ws[TK][TN + 1];
  __shared__ float Cs[TM][TN + 1];
  const T *A = (const T *)a.A;
  const T *W = (const T *)a.W;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += TK) {
    for (int e = tid; e < TM * TK; e += 256) {
      const int r = e / TK, c = e % TK;
      const int gm = m0 + r, gk = k0 + c;
      As[c][r] = (gm < a.M && gk < a.K) ? to_f32(A[(int64_t)gm * a.lda + gk]) : 0.f;
      const int gn = n0 + r;
      Ws[c][r] = (gn < a.N && gk < a.K) ? to_f32(W[(int64_t)gn * a.K + gk]) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < TK; ++k) {
      float av[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = Ws[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
  if (a.epi == Epi::SwiGLU) {
    // The tile's 64 packed rows are two (gate block, up block) pairs.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) Cs[ty + 16 * i][tx + 16 * j] = acc[i][j] * a.scale;
    __syncthreads();
    T *out = (T *)a.act_out;
    for (int e = tid; e < TM * (TN / 2); e += 256) {
      const int r = e / (TN / 2), f = e % (TN / 2);
      const int pair = f / GU_BLOCK, w = f % GU_BLOCK;
      const int gm = m0 + r, gf = n0 / 2 + f;
      if (gm < a.M && gf < a.N / 2) {
        const float g = Cs[r][pair * 2 * GU_BLOCK + w];
        const float u = Cs[r][pair * 2 * GU_BLOCK + GU_BLOCK + w];
        out[(int64_t)gm * a.ldo + gf] = from_f32<T>(silu_f(g) * u);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty + 16 * i;
    if (gm >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx + 16 * j;
      if (gn >= a.N) continue;
      float *o = a.out_f32 + (int64_t)gm * a.ldo + gn;
      if (a.epi == Epi::ResidAdd)
        *o += acc[i][j] * a.scale;
      else
        *o = acc[i][j] * a.scale;
    }
  }
}
}  // namespace

hipError_t launch_gemm_generic(hipStream_t s, bool f16_mode, const GemmArgs &a) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  dim3 grid((a.N + TN - 1) / TN, (a.M + TM - 1) / TM);
  if (f16_mode)
    QW_LAUNCH((gemm_generic_kernel<f16>), dim3(grid), dim3(256), 0, s, a);
  else
    QW_LAUNCH((gemm_generic_kernel<float>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qw
