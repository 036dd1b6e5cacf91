// Window scoring: dispatch to the kernel instantiated per dtype and head
// size (kara_score_kernel.hpp), and the reduction of per-chunk partial sums
// used by the stand-alone scoring entry point.

#include "kara_internal.hpp"

namespace kara {

template <typename T, int D>
hipError_t launch_score_typed(const ScoreArgs& a, hipStream_t stream);

namespace {

__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ partials,
                                                     float* __restrict__ scores, int n_units,
                                                     int n_split, int C) {
  const size_t n = (size_t)n_units * C;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t u = i / C, j = i - (i / C) * C;
    const float* p = partials + u * n_split * C + j;
    // chunks read eight at a time (loads issued before any add), added in order
    float s = 0.0f;
    for (int k0 = 0; k0 < n_split; k0 += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = k0 + k < n_split ? p[(size_t)(k0 + k) * C] : 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k0 + k < n_split) s += v[k];
    }
    scores[i] = s;
  }
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream) {
  if (a.n_units == 0) return hipSuccess;
  if (use_resident(dtype, a.D, a.W, a.G, a.unidirectional)) {
    if (a.n_split != 1) return hipErrorInvalidValue;
    return launch_score_resident(a, stream);
  }
  if (dtype == 1) {
    if (a.D == 128) return launch_score_typed<__bf16, 128>(a, stream);
    if (a.D == 64) return launch_score_typed<__bf16, 64>(a, stream);
  } else {
    if (a.D == 128) return launch_score_typed<float, 128>(a, stream);
    if (a.D == 64) return launch_score_typed<float, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const float* partials, float* scores, int n_units, int n_split, int C,
                         hipStream_t stream) {
  if (n_units == 0) return hipSuccess;
  const size_t n = (size_t)n_units * C;
  unsigned grid = (unsigned)((n + 255) / 256);
  if (grid > 65536u) grid = 65536u;
  hipLaunchKernelGGL(reduce_kernel, dim3(grid), dim3(256), 0, stream, partials, scores, n_units,
                     n_split, C);
  return hipGetLastError();
}

}  // namespace kara
