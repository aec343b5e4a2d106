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

// Streaming HBM probe: 16 bytes per lane, UNROLL accesses in flight per
// lane, grid-stride over the buffer.  MODE 0 copies src to dst, 1 only reads
// src (a per-thread checksum goes to dst[thread]), 2 only writes dst.
constexpr int kStreamUnroll = 4;

template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void stream_probe_kernel(const uint4 *__restrict__ src,
                                                                    uint4 *__restrict__ dst,
                                                                    int64_t n16) {
  const int64_t nthr = (int64_t)gridDim.x * kProbeThreads;
  const int64_t t = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t sum = 0;
  for (int64_t i = t; i < n16; i += nthr * kStreamUnroll) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) {
      const int64_t j = i + k * nthr;
      if (MODE == 2) v[k] = make_uint4((uint32_t)j, 1u, 2u, 3u);
      else if (j < n16) v[k] = src[j];
    }
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) {
      const int64_t j = i + k * nthr;
      if (j < n16) {
        if (MODE == 1) sum += v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
        else dst[j] = v[k];
      }
    }
  }
  if (MODE == 1) reinterpret_cast<uint32_t *>(dst)[t] = sum;
}

}  // namespace lh

extern "C" lh_status lh_probe_stream(int32_t mode, const void *src, void *dst, size_t bytes,
                                     int64_t blocks, lh_stream stream) {
  if (mode < 0 || mode > 2 || bytes == 0 || bytes % 16 || !dst || (mode != 2 && !src) ||
      !lh::grid_fits(blocks, lh::kProbeThreads) || blocks <= 0 ||
      ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
    return LH_ERR_INVALID_ARG;
  (void)hipGetLastError();   // report this launch's error only
  const int64_t n16 = (int64_t)(bytes / 16);
  const uint4 *s = (const uint4 *)src;
  uint4 *d = (uint4 *)dst;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)blocks), blk(lh::kProbeThreads);
  if (mode == 0) hipLaunchKernelGGL(lh::stream_probe_kernel<0>, grid, blk, 0, st, s, d, n16);
  else if (mode == 1) hipLaunchKernelGGL(lh::stream_probe_kernel<1>, grid, blk, 0, st, s, d, n16);
  else hipLaunchKernelGGL(lh::stream_probe_kernel<2>, grid, blk, 0, st, s, d, n16);
  return lh::hip_status();
}

extern "C" lh_status lh_probe_mfma_bf16(int64_t blocks, int32_t iters, float *out,
                                        lh_stream stream) {
  if (!lh::grid_fits(blocks, lh::kProbeThreads) || blocks <= 0 || iters <= 0 || !out)
    return LH_ERR_INVALID_ARG;
  (void)hipGetLastError();   // report this launch's error only
  hipLaunchKernelGGL(lh::mfma_probe_kernel, dim3((unsigned)blocks), dim3(lh::kProbeThreads), 0,
                     (hipStream_t)stream, out, iters);
  return lh::hip_status();
}
