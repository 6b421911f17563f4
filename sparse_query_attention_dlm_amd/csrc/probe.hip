// Measured MFMA ceiling of this GPU (a measurement aid, not a step of the
// method): every wave keeps eight independent chains of 32x32x16 bf16 MFMAs
// on register operands busy for `iters` rounds, with no memory traffic, so
// the achieved rate is the matrix pipes' peak at the clock the chip holds
// under full MFMA load.  Rooflines are reported against this figure as well
// as against the published peak.
#include "common.hpp"
#include "launch.hpp"

namespace dlm {

constexpr int kProbeChains = 8;

__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  // lane-dependent operands, so that nothing is known at compile time
  u32x4 wa, wb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wa[j] = pack_bf16x2(1.f + 1e-3f * lane, 1.f - 1e-3f * j);
    wb[j] = pack_bf16x2(1e-3f * j, 1e-3f * lane);
  }
  const bf16x8 a = as_bf16x8(wa), b = as_bf16x8(wb);
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma32x32x16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_probe_mfma(int iters, int grid, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(grid), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

}  // namespace dlm
