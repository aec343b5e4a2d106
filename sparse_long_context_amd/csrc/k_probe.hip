// Measurement helper: the issue rate this device sustains for the bf16 MFMA
// the attention kernels use (v_mfma_f32_32x32x16_bf16), from independent
// accumulation chains with no memory traffic.  The roofline's published
// peak is an upper bound the clock does not hold under sustained MFMA load;
// this gives the achievable ceiling beside it.
#include "lh_mfma.h"

namespace lh {

constexpr int kProbeChains = 8;
constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float *out, int32_t iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(2e-3f * (float)i);
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;   // keeps the chains live
}

}  // namespace lh

extern "C" lh_status lh_probe_mfma_bf16(int64_t blocks, int32_t iters, float *out,
                                        lh_stream stream) {
  if (!lh::grid_fits(blocks, lh::kProbeThreads) || blocks <= 0 || iters <= 0 || !out)
    return LH_ERR_INVALID_ARG;
  (void)hipGetLastError();   // report this launch's error only
  hipLaunchKernelGGL(lh::mfma_probe_kernel, dim3((unsigned)blocks), dim3(lh::kProbeThreads), 0,
                     (hipStream_t)stream, out, iters);
  return lh::hip_status();
}
