// Kronecker layer loss tr(dW H_X dW^T H_G), dW = W^ - W, in float64.
//
// The loss is the quadratic form of the Kronecker-factored Hessian H_X kron H_G
// on vec(dW) ("KronQ: LLM Quantization via Kronecker-Factored Hessian",
// gptget.net, Abstract; aimodeling.com news item: H ~ H_X kron H_G). With
// P = dW H_X and Q = H_G dW (both dout x din) it equals the sum over all
// entries of P * Q, so every 64 x 64 output tile is independent:
//   1. diff_kernel: dW = W^ - W in float64 (W bf16, float32 or float64);
//   2. tile_kernel: one workgroup per 64 x 64 tile forms its tile of P and
//      of Q on float64 MFMA (v_mfma_f64_16x16x4f64, k in chunks of 16 through
//      LDS) and writes sum(P * Q) over the tile as one partial;
//   3. sum_kernel: one workgroup adds the partials in a fixed order.
// Every sum has a fixed order, so the result is the same on every run.
#include "kq_internal.h"

namespace kq {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 64;      // output tile edge
constexpr int kK = 16;      // k chunk
constexpr int kPad = kT + 2;

template <typename T>
__device__ __forceinline__ double ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ double ld<uint16_t>(const uint16_t* p, int64_t i) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(p[i]) << 16));
}
template <>
__device__ __forceinline__ double ld<float>(const float* p, int64_t i) {
  return static_cast<double>(p[i]);
}
template <>
__device__ __forceinline__ double ld<double>(const double* p, int64_t i) {
  return p[i];
}

template <typename TW>
__global__ void diff_kernel(const double* __restrict__ w_hat, const TW* __restrict__ w, int64_t n,
                            double* __restrict__ dw) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dw[i] = w_hat[i] - ld<TW>(w, i);
}

struct TileLds {
  double a[2][kK][kPad];  // [k][row]
  double b[2][kK][kPad];  // [k][column]
};

// acc (this wave's 32 x 32 quarter of a 64 x 64 tile, as 2 x 2 MFMA blocks) = A[i0.., :] B[:, j0..]
// over k < K: A element (i, k) at a[i * lda + k], B element (k, j) at b[k * ldb + j]. Rows past M
// and columns past N read as zero.
template <typename TA, typename TB>
__device__ __forceinline__ void tile_product(TileLds& sm, const TA* __restrict__ a, int64_t lda,
                                             const TB* __restrict__ b, int64_t ldb, int64_t K, int64_t M,
                                             int64_t N, int64_t i0, int64_t j0, f64x4 (&acc)[2][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{};
  // loads of one chunk: 64 x 16 of A (4 per thread) and 16 x 64 of B (4 per thread)
  double va[4], vb[4];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int ar = e >> 4, ak = e & 15;       // A: row ar, k ak (k fastest: rows are contiguous in k)
      const int64_t gi = i0 + ar, gk = k0 + ak;
      va[q] = (gi < M && gk < K) ? ld<TA>(a, gi * lda + gk) : 0.0;
      const int bk = e >> 6, bj = e & 63;       // B: k bk, column bj (columns contiguous)
      const int64_t gk2 = k0 + bk, gj = j0 + bj;
      vb[q] = (gk2 < K && gj < N) ? ld<TB>(b, gk2 * ldb + gj) : 0.0;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      sm.a[buf][e & 15][e >> 4] = va[q];
      sm.b[buf][e >> 6][e & 63] = vb[q];
    }
  };
  const int64_t nch = (K + kK - 1) / kK;
  load(0);
  store(0);
  __syncthreads();
  const int il = lane & 15, kl = lane >> 4;
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int buf = static_cast<int>(ch & 1);
    if (ch + 1 < nch) load((ch + 1) * kK);
#pragma unroll
    for (int kk = 0; kk < kK / 4; ++kk) {
      const int kr = 4 * kk + kl;
      double fa[2], fb[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) fa[x] = sm.a[buf][kr][wi * 32 + x * 16 + il];
#pragma unroll
      for (int y = 0; y < 2; ++y) fb[y] = sm.b[buf][kr][wj * 32 + y * 16 + il];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    if (ch + 1 < nch) store(buf ^ 1);
    __syncthreads();
  }
}

// Partial of tile t: sum over the tile of (dW H_X) * (H_G dW).
__global__ __launch_bounds__(256) void tile_kernel(const double* __restrict__ dw, const float* __restrict__ hx,
                                                   const float* __restrict__ hg, int64_t dout, int64_t din,
                                                   int64_t tiles_j, double* __restrict__ partial) {
  __shared__ TileLds sm;
  __shared__ double red[4];
  const int64_t t = blockIdx.x;
  const int64_t i0 = (t / tiles_j) * kT, j0 = (t % tiles_j) * kT;
  f64x4 p[2][2], q[2][2];
  tile_product<double, float>(sm, dw, din, hx, din, din, dout, din, i0, j0, p);   // P = dW H_X
  tile_product<float, double>(sm, hg, dout, dw, din, dout, dout, din, i0, j0, q);  // Q = H_G dW
  // the two products share one register layout, so P * Q pairs up entry by entry
  double s = 0.0;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) s = fma(p[x][y][r], q[x][y][r], s);
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) partial[t] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void sum_kernel(const double* __restrict__ partial, int64_t n,
                                                  double* __restrict__ loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += partial[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = red[0];
}

struct Layout {
  int64_t tiles_i, tiles_j;
  size_t dw_bytes, part_bytes;
};

Layout layout(int64_t dout, int64_t din) {
  Layout l{};
  l.tiles_i = (dout + kT - 1) / kT;
  l.tiles_j = (din + kT - 1) / kT;
  l.dw_bytes = align_up(size_t(dout) * din * sizeof(double), 256);
  l.part_bytes = align_up(size_t(l.tiles_i * l.tiles_j) * sizeof(double), 256);
  return l;
}

}  // namespace

size_t loss_workspace(int64_t dout, int64_t din) {
  const Layout l = layout(dout, din);
  return l.dw_bytes + l.part_bytes;
}

kq_status loss_run(const double* w_hat, const void* w, int w_dtype, int64_t dout, int64_t din, const float* h_x,
                   const float* h_g, double* loss, void* ws, hipStream_t st) {
  const Layout l = layout(dout, din);
  double* dw = static_cast<double*>(ws);
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + l.dw_bytes);
  const int64_t n = dout * din;
  const unsigned nb = static_cast<unsigned>((n + 255) / 256);
  {
    LaunchTimer timer("loss_diff_kernel", st);
    if (w_dtype == KQ_BF16)
      hipLaunchKernelGGL(diff_kernel<uint16_t>, dim3(nb), dim3(256), 0, st, w_hat, static_cast<const uint16_t*>(w), n, dw);
    else if (w_dtype == KQ_F32)
      hipLaunchKernelGGL(diff_kernel<float>, dim3(nb), dim3(256), 0, st, w_hat, static_cast<const float*>(w), n, dw);
    else
      hipLaunchKernelGGL(diff_kernel<double>, dim3(nb), dim3(256), 0, st, w_hat, static_cast<const double*>(w), n, dw);
  }
  kq_status s = check_launch("loss_diff_kernel");
  if (s != KQ_OK) return s;
  const int64_t ntiles = l.tiles_i * l.tiles_j;
  {
    LaunchTimer timer("loss_tile_kernel", st);
    hipLaunchKernelGGL(tile_kernel, dim3(static_cast<unsigned>(ntiles)), dim3(256), 0, st, dw, h_x, h_g, dout, din,
                       l.tiles_j, part);
  }
  if ((s = check_launch("loss_tile_kernel")) != KQ_OK) return s;
  {
    LaunchTimer timer("loss_sum_kernel", st);
    hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(256), 0, st, part, ntiles, loss);
  }
  return check_launch("loss_sum_kernel");
}

}  // namespace kq
