// Opt-in check of a selection's index arrays (DLM_VALIDATE=1 in the
// environment): the calls that scatter rows into the caches trust idx and
// offsets, so an index past the sequence, an unordered row or inconsistent
// offsets would make them write outside the caller's tensors.  With the check
// on, each such call first runs this kernel, reads its verdict back (the call
// then synchronises with the host) and returns DLM_ERR_INVALID_ARG before any
// other launch when the arrays break the selection format: offsets[0] = 0,
// offsets non-decreasing, offsets[B] <= max_rows, and within each batch row
// positions strictly increasing and inside [0, S).
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace dlm {

// the verdict of the last check on this GPU (one word per GPU; checks are
// serialised by the host-side mutex below)
static __device__ int validate_status;

// One workgroup: the offsets first, then (only when they are consistent, so
// that every row's batch row is well defined) every selected position.
__global__ __launch_bounds__(1024) void validate_rows_kernel(const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ offsets,
                                                             int B, int S, int max_rows,
                                                             int check_idx, int* status) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int f = 0;
  if (threadIdx.x == 0) {
    if (offsets[0] != 0) f |= kBadFirstOffset;
    if (offsets[B] > max_rows) f |= kOffsetsPastBound;
  }
  for (int b = threadIdx.x; b < B; b += blockDim.x)
    if (offsets[b + 1] < offsets[b]) f |= kOffsetsDecrease;
  if (f) atomicOr(&flags, f);
  __syncthreads();
  if (check_idx && flags == 0) {
    f = 0;
    const int n = offsets[B];
    for (int r = threadIdx.x; r < n; r += blockDim.x) {
      const int b = batch_of(offsets, B, r);
      const int i = idx[r];
      if (i < 0 || i >= S) f |= kIndexOutside;
      if (r > offsets[b] && idx[r - 1] >= i) f |= kIndexOrder;
    }
    if (f) atomicOr(&flags, f);
    __syncthreads();
  }
  if (threadIdx.x == 0) *status = flags;
}

hipError_t validate_rows(const int32_t* idx, const int32_t* offsets, int B, int S, int max_rows,
                         int check_idx, hipStream_t st, int* verdict) {
  static std::mutex mu;
  static int* ptrs[64] = {};
  *verdict = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(validate_status));
    if (e != hipSuccess) return e;
    ptrs[dev] = static_cast<int*>(p);
  }
  hipLaunchKernelGGL(validate_rows_kernel, dim3(1), dim3(1024), 0, st, idx, offsets, B, S, max_rows,
                     check_idx, ptrs[dev]);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int v = 0;
  e = hipMemcpyAsync(&v, ptrs[dev], sizeof(int), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  *verdict = v;
  return hipSuccess;
}

}  // namespace dlm
