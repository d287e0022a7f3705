// Measured peaks for the roofline fractions: an HBM copy and an MFMA-only
// loop, timed on the caller's stream.  Neither is on the forward pass; they
// give the denominators a run can actually reach beside the published ones
// (8 TB/s HBM, 2.5 PFLOP/s dense fp16 on the MI355X).
#include "../../include/qw.h"
#include "qw_internal.h"


// Written only on an impossible value of the MFMA loop's result, so the
// compiler keeps the loop (external linkage: the store cannot be dropped).
__device__ float qw_peak_sink;

namespace qw {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Grid-stride over n 16-byte elements, kUnroll loads issued per lane before
// any is used.  Copy: dst = src.  Read: every element is read once and each
// thread writes one 16-byte combination of what it read (to dst[thread]), so
// the written bytes are negligible next to the read ones.
constexpr int kUnroll = 4;
__global__ void __launch_bounds__(256) peak_copy_kernel(float4 *__restrict__ dst, const float4 *__restrict__ src,
                                                        int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    float4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// CONTIG: a thread's kUnroll loads are consecutive (64 bytes, a wave covers
// 4 KB at once); otherwise they are a grid apart (a wave covers 1 KB per load).
template <bool CONTIG>
__global__ void __launch_bounds__(256) peak_read_kernel(float4 *__restrict__ dst, const float4 *__restrict__ src,
                                                        int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = CONTIG ? 1 : stride;
  int64_t i = CONTIG ? ((int64_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x * kUnroll) : t;
  const int64_t adv = kUnroll * stride;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (; i + (kUnroll - 1) * step < n; i += adv) {
    float4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * step];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
  }
  // n is a multiple of kUnroll * stride in every use (the host requires
  // bytes to be a multiple of 64 MiB), so only the grid-apart layout could
  // have a partial round
  if (!CONTIG) {
    for (; i < n; i += stride) {
      const float4 v = src[i];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
  }
  dst[t] = acc;
}

// Each wave issues `iters` rounds of kChains independent 16x16x32 fp16
// products on register operands (independent accumulators hide the
// dependent-issue latency).  Only the matrix cores work inside the loop.
constexpr int kChains = 8;
__global__ void __launch_bounds__(256) peak_mfma_kernel(int iters) {
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(1e-3f * (float)((threadIdx.x + e) & 7));
    b[e] = (_Float16)(1e-3f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == -1.2345e-30f) qw_peak_sink = s;     // never true for these operands; keeps the loop
}

constexpr int kMfmaWorkgroups = 2048;       // 8 per CU: 8 waves per SIMD, all resident at once
constexpr double kMfmaFlopPerWaveIter = 2.0 * 16 * 16 * 32 * kChains;

}  // namespace
}  // namespace qw

using namespace qw;

namespace {

// Runs `launch` between two events on `s` and returns the elapsed ms.
template <class F>
hipError_t time_on_stream(hipStream_t s, F &&launch, float *ms) {
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) e = hipEventRecord(a, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  return e;
}

}  // namespace

extern "C" {

qw_status qw_peak_copy(void *dst, const void *src, int64_t bytes, int32_t iters, int32_t read_only,
                       void *hip_stream, double *gbs) {
  clear_error();
  constexpr int kBlocks = 256 * 8;          // 8 workgroups per CU, grid-stride over the rest
  if (!dst || !src || !gbs || bytes % (64 << 20) != 0 || iters < 1)
    return (qw_status)report(QW_ERR_INVALID_ARG, "qw_peak_copy: need device pointers, bytes a positive multiple of "
                                                 "64 MiB, iters >= 1 and an output");
  hipStream_t s = (hipStream_t)hip_stream;
  const int64_t n = bytes / 16;
  if (!read_only) {
    float ms = 0.f;
    hipError_t e = time_on_stream(s, [&] {
      for (int i = 0; i < iters; ++i)
        hipLaunchKernelGGL(peak_copy_kernel, dim3(kBlocks), dim3(256), 0, s, (float4 *)dst, (const float4 *)src, n);
      return hipGetLastError();
    }, &ms);
    if (e != hipSuccess) return (qw_status)report(QW_ERR_HIP, "qw_peak_copy: %s", hipGetErrorString(e));
    *gbs = 2.0 * (double)bytes * iters / (ms * 1e-3) / 1e9;
    return QW_OK;
  }
  // reads: the best of both load layouts at 4, 8 and 16 workgroups per CU
  // (every configuration writes at most dst[0 .. 16 * 256 * 256))
  double best = 0.0;
  for (int layout = 0; layout < 2; ++layout)
    for (int per_cu = 4; per_cu <= 16; per_cu *= 2) {
      const int blocks = 256 * per_cu;
      float ms = 0.f;
      hipError_t e = time_on_stream(s, [&] {
        for (int i = 0; i < iters; ++i) {
          if (layout)
            hipLaunchKernelGGL(peak_read_kernel<true>, dim3(blocks), dim3(256), 0, s, (float4 *)dst, (const float4 *)src, n);
          else
            hipLaunchKernelGGL(peak_read_kernel<false>, dim3(blocks), dim3(256), 0, s, (float4 *)dst, (const float4 *)src, n);
        }
        return hipGetLastError();
      }, &ms);
      if (e != hipSuccess) return (qw_status)report(QW_ERR_HIP, "qw_peak_copy: %s", hipGetErrorString(e));
      const double r = (double)bytes * iters / (ms * 1e-3) / 1e9;
      if (r > best) best = r;
    }
  *gbs = best;
  return QW_OK;
}

qw_status qw_peak_mfma(int32_t iters, void *hip_stream, double *tflops) {
  clear_error();
  if (!tflops || iters < 1) return (qw_status)report(QW_ERR_INVALID_ARG, "qw_peak_mfma: iters >= 1 and an output");
  hipStream_t s = (hipStream_t)hip_stream;
  float ms = 0.f;
  hipError_t e = time_on_stream(s, [&] {
    hipLaunchKernelGGL(peak_mfma_kernel, dim3(kMfmaWorkgroups), dim3(256), 0, s, iters);
    return hipGetLastError();
  }, &ms);
  if (e != hipSuccess) return (qw_status)report(QW_ERR_HIP, "qw_peak_mfma: %s", hipGetErrorString(e));
  const double waves = (double)kMfmaWorkgroups * 4;
  *tflops = waves * iters * kMfmaFlopPerWaveIter / (ms * 1e-3) / 1e12;
  return QW_OK;
}

}  // extern "C"
