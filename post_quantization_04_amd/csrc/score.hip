// Sub-layer sensitivity tr(H_G) * tr(H_X) (or tr(H_X) alone) in float64.
//
// One workgroup walks both diagonals with a fixed thread-to-element mapping
// and a fixed reduction tree, so the score is bit-reproducible run to run.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kThreads = 256;

__device__ double block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void score_kernel(const float* __restrict__ h_x, int64_t din,
                                                         const float* __restrict__ h_g, int64_t dout,
                                                         int mode, double* __restrict__ score) {
  __shared__ double red[kThreads];
  double sx = 0.0;
  for (int64_t i = threadIdx.x; i < din; i += kThreads) sx += static_cast<double>(h_x[i * din + i]);
  const double tx = block_sum(sx, red);
  double out = tx;
  if (mode == KQ_SCORE_KRONQ) {
    double sg = 0.0;
    for (int64_t i = threadIdx.x; i < dout; i += kThreads) sg += static_cast<double>(h_g[i * dout + i]);
    out = block_sum(sg, red) * tx;
  }
  if (threadIdx.x == 0) *score = out;
}

}  // namespace

kq_status score_run(const float* h_x, int64_t din, const float* h_g, int64_t dout, int mode, double* score,
                    hipStream_t st) {
  {
    LaunchTimer timer("score_kernel", st);
    hipLaunchKernelGGL(score_kernel, dim3(1), dim3(kThreads), 0, st, h_x, din, h_g, dout, mode, score);
  }
  return check_launch("score_kernel");
}

}  // namespace kq
