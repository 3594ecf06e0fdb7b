// Upper-triangular R with R^T R = (H + damp * mean(diag H) * I)^-1.
//
// With J the index-reversal permutation, J H~ J = L L^T (lower Cholesky) gives
// H~ = V V^T with V = J L J upper, and R = V^-1 = J L^-1 J. So the kernel
// chain is:
//   1. damping: delta = damp * mean(diag H) in float64;
//   2. reversal copy A = J H J + delta I into scratch, padded to a multiple of
//      64 with an identity block;
//   3. blocked right-looking Cholesky of A with 64 x 64 blocks: the diagonal
//      block is factored (and inverted) in float64 in LDS by one workgroup,
//      the panel below it is multiplied by the inverse block, and the
//      trailing lower triangle receives the rank-64 update, both on float32
//      MFMA (v_mfma_f32_32x32x2f32);
//   4. M = L^-1 by recursive doubling: diagonal blocks are already inverted;
//      at each level, neighbouring blocks (B1, B2) merge with
//      M21 = -M22 (L21 M11), two batched MFMA products that skip the zero
//      triangles of M11 and M22;
//   5. R = J M J written over H (strict lower triangle zeroed).
// A pivot that is not positive and finite stops the chain: `info` takes the
// original index + 1 and every later kernel returns at once.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kB = 64;  // block edge

typedef float f32x16 __attribute__((ext_vector_type(16)));

// --------------------------------------------------------------------------
// 64 x 64 float32 MFMA tile product: C = alpha * A B + beta * C over k in [k0, k1)
//   A element (i, k) at a[i * lda + k] (TA: a[k * lda + i])
//   B element (k, j) at b[k * ldb + j] (TB: b[j * ldb + k])
// C may alias A (the panel step): every load of A precedes the first store.
// m_valid / n_valid bound the tile; k beyond k1 reads as zero.
// 256 threads: 4 waves in a 2 x 2 grid of 32 x 32 blocks.
// --------------------------------------------------------------------------
template <bool TA, bool TB>
__device__ void gemm_tile(const float* a, int64_t lda, const float* b, int64_t ldb, float* c, int64_t ldc, int m_valid, int n_valid, int k0, int k1,
                          float alpha, float beta) {
  __shared__ float as[32][kB + 4];
  __shared__ float bs[32][kB + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  f32x16 acc = f32x16{};
  for (int kc = k0; kc < k1; kc += 32) {
    // stage A (64 x 32) and B (32 x 64)
    for (int e = tid; e < kB * 32; e += 256) {
      int i, k;
      if (TA) { i = e & 63; k = e >> 6; } else { k = e & 31; i = e >> 5; }
      const int kg = kc + k;
      as[k][i] = (i < m_valid && kg < k1) ? (TA ? a[int64_t(kg) * lda + i] : a[int64_t(i) * lda + kg]) : 0.0f;
      int j, k2;
      if (TB) { k2 = e & 31; j = e >> 5; } else { j = e & 63; k2 = e >> 6; }
      const int kg2 = kc + k2;
      bs[k2][j] = (j < n_valid && kg2 < k1) ? (TB ? b[int64_t(j) * ldb + kg2] : b[int64_t(kg2) * ldb + j]) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float fa = as[2 * kk + (lane >> 5)][wi * 32 + (lane & 31)];
      const float fb = bs[2 * kk + (lane >> 5)][wj * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa, fb, acc, 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = wi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int j = wj * 32 + (lane & 31);
    if (i < m_valid && j < n_valid) {
      float* p = c + int64_t(i) * ldc + j;
      *p = (beta == 0.0f) ? alpha * acc[r] : alpha * acc[r] + beta * *p;
    }
  }
}

__device__ __forceinline__ void tri(int t, int& I, int& J) {
  int i = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  I = i;
  J = t - i * (i + 1) / 2;
}

__global__ __launch_bounds__(256) void damp_kernel(const float* __restrict__ h, int64_t d, float damp,
                                                   double* __restrict__ delta, int32_t* __restrict__ info) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256) s += static_cast<double>(h[i * d + i]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *delta = static_cast<double>(damp) * red[0] / static_cast<double>(d);
    *info = 0;
  }
}

// A[i][j] = H[d-1-i][d-1-j] + delta [i == j]; identity outside d.
__global__ void reverse_kernel(const float* __restrict__ h, int64_t d, int64_t dp, const double* __restrict__ delta,
                               float* __restrict__ a) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t i = blockIdx.y;
  if (j >= dp) return;
  float v;
  if (i < d && j < d) {
    v = h[(d - 1 - i) * d + (d - 1 - j)];
    if (i == j) v = static_cast<float>(static_cast<double>(v) + *delta);
  } else {
    v = (i == j) ? 1.0f : 0.0f;
  }
  a[i * dp + j] = v;
}

// ---------------------------------------------------------------------------
// Diagonal block factorization in float64 with 16 x 16 sub-blocks.
//   * base cases (16 x 16 Cholesky and its inverse) run on one wave, lanes
//     0..15 owning one row each in registers, columns broadcast through LDS;
//   * sub-panel, trailing and inverse products are float64 MFMA 16 x 16 x 4
//     (operands A[i][k] at lane i + 16 k, B[k][j] at lane j + 16 k; result
//     row 4 q + lane / 16, column lane % 16 in register q).
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kP = kB + 1;  // LDS row pitch (doubles)

// acc += A16 * B16 (or A16 * B16^T) for 16 x 16 tiles in LDS with pitch kP; one wave.
template <bool BT>
__device__ __forceinline__ f64x4 mm16(const double* a, const double* b, f64x4 acc) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const double fa = a[r * kP + 4 * kk + c];
    const double fb = BT ? b[r * kP + 4 * kk + c] : b[(4 * kk + c) * kP + r];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(fa, fb, acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ void store16(double* c, f64x4 v, double scale) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) c[(4 * q + (lane >> 4)) * kP + (lane & 15)] = scale * v[q];
}

__device__ __forceinline__ f64x4 load16(const double* c) {
  const int lane = threadIdx.x & 63;
  f64x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = c[(4 * q + (lane >> 4)) * kP + (lane & 15)];
  return v;
}

// Value of v in lane `src` (a compile-time lane), for every lane.
__device__ __forceinline__ double bcast(double v, int src) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(b), src));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), src));
  return __builtin_bit_cast(double, (static_cast<unsigned long long>(hi) << 32) | lo);
}

// 1 / sqrt(p) for finite p > 0: the hardware estimate refined by two Newton
// steps y <- y + y (1 - p y^2) / 2, which brings it to float64 rounding.
__device__ __forceinline__ double rsqrt_f64(double p) {
  double y = __builtin_amdgcn_rsq(p);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = fma(-p * y, y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return y;
}

// 16 x 16 Cholesky (lower) of the sub-block at l + o * (kP + 1) and its inverse
// into x + o * (kP + 1); wave 0 only. Lane i < 16 holds row i in registers;
// columns are broadcast with readlane and pivots use 1 / sqrt(p), so the
// column chain has no division, square root or LDS round trip. Returns the
// local index of the first bad pivot, or -1.
__device__ int base16(double* l, double* x, int o) {
  const int lane = threadIdx.x & 63;
  const bool act = lane < 16;
  double* L = l + o * (kP + 1);
  double* X = x + o * (kP + 1);
  double r[16], y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) r[j] = act ? L[lane * kP + j] : 0.0;
  // Factor: after step k, lanes i >= k hold l_ik in r[k]. Lanes i < j also
  // update their (upper) r[j]; those values are never broadcast and are
  // cleared when their column comes up.
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const double p = bcast(r[k], k);
    if (!(p > 0.0) || !(p < __builtin_huge_val())) return k;  // uniform
    y[k] = rsqrt_f64(p);
    const double lik = (lane == k) ? p * y[k] : r[k] * y[k];
    r[k] = (lane >= k) ? lik : 0.0;
#pragma unroll
    for (int j = k + 1; j < 16; ++j) r[j] = fma(-lik, bcast(lik, j), r[j]);
  }
  // Inverse by forward substitution: lane i holds row i of X = L^-1. At step
  // k row k is scaled by 1 / l_kk = y_k, then removed from the rows below.
  double xr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) xr[j] = (lane == j) ? 1.0 : 0.0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
#pragma unroll
    for (int j = 0; j <= k; ++j) xr[j] = (lane == k) ? xr[j] * y[k] : xr[j];
    const double lik = (lane > k) ? r[k] : 0.0;
#pragma unroll
    for (int j = 0; j <= k; ++j) xr[j] = fma(-lik, bcast(xr[j], k), xr[j]);
  }
  if (act) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      L[lane * kP + j] = (j <= lane) ? r[j] : 0.0;
      X[lane * kP + j] = (j <= lane) ? xr[j] : 0.0;
    }
  }
  return -1;
}

// Factor the 64 x 64 diagonal block kb (float64), invert its factor, and solve
// one 64-row block of the panel below it: workgroup 0 writes L_kk to A and
// L_kk^-1 to M; workgroup b >= 1 writes L[kb + b, kb] = A[kb + b, kb] L_kk^-T.
// Every workgroup factors the (small) diagonal block itself.
__global__ __launch_bounds__(256) void diag_panel_kernel(float* __restrict__ a, float* __restrict__ m, int64_t dp,
                                                         int kb, int64_t d, int32_t* __restrict__ info) {
  __shared__ double l[kB * kP];
  __shared__ double x[kB * kP];
  __shared__ int bad;
  if (*info) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t o = int64_t(kb) * kB;
  for (int e = tid; e < kB * kB; e += 256) {
    const int i = e >> 6, j = e & 63;
    l[i * kP + j] = (j <= i) ? static_cast<double>(a[(o + i) * dp + o + j]) : 0.0;
    x[i * kP + j] = 0.0;
  }
  if (tid == 0) bad = -1;
  __syncthreads();
  for (int s = 0; s < 4; ++s) {
    if (wave == 0) {
      const int b = base16(l, x, 16 * s);
      if (lane == 0 && b >= 0) bad = 16 * s + b;
    }
    __syncthreads();
    if (bad >= 0) {
      if (tid == 0 && blockIdx.x == 0) {
        const int64_t ir = o + bad;
        atomicCAS(info, 0, static_cast<int32_t>(((ir < d) ? d - 1 - ir : ir) + 1));
      }
      return;
    }
    // sub-panel: L[t][s] = A[t][s] inv(L_ss)^T for t > s (one tile per wave)
    const int t = s + 1 + wave;
    f64x4 v = f64x4{};
    if (t < 4) v = mm16<true>(l + 16 * t * kP + 16 * s, x + 16 * s * kP + 16 * s, v);
    __syncthreads();
    if (t < 4) store16(l + 16 * t * kP + 16 * s, v, 1.0);
    __syncthreads();
    // trailing: A[t][u] -= L[t][s] L[u][s]^T for s < u <= t (at most 6 tiles)
    for (int q = wave; q < 6; q += 4) {
      int tt = 0, uu = 0, n = 0;
      for (int ti = s + 1; ti < 4; ++ti)
        for (int ui = s + 1; ui <= ti; ++ui, ++n)
          if (n == q) { tt = ti; uu = ui; }
      if (q < n) {
        f64x4 c = load16(l + 16 * tt * kP + 16 * uu);
        f64x4 p = mm16<true>(l + 16 * tt * kP + 16 * s, l + 16 * uu * kP + 16 * s, f64x4{});
        store16(l + 16 * tt * kP + 16 * uu, c - p, 1.0);
      }
    }
    __syncthreads();
  }
  // inverse: M[t][s] = -inv(L_tt) sum_{u = s}^{t - 1} L[t][u] M[u][s], row block by row block
  for (int t = 1; t < 4; ++t) {
    const int s = wave;  // one column block per wave
    f64x4 acc = f64x4{};
    if (s < t) {
      for (int u = s; u < t; ++u) acc = mm16<false>(l + 16 * t * kP + 16 * u, x + 16 * u * kP + 16 * s, acc);
    }
    __syncthreads();
    if (s < t) store16(x + 16 * t * kP + 16 * s, acc, 1.0);  // temporary: T = sum L M
    __syncthreads();
    f64x4 mv = f64x4{};
    if (s < t) mv = mm16<false>(x + 16 * t * kP + 16 * t, x + 16 * t * kP + 16 * s, f64x4{});
    __syncthreads();
    if (s < t) store16(x + 16 * t * kP + 16 * s, mv, -1.0);
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    for (int e = tid; e < kB * kB; e += 256) {
      const int i = e >> 6, j = e & 63;
      if (j <= i) a[(o + i) * dp + o + j] = static_cast<float>(l[i * kP + j]);
      m[(o + i) * dp + o + j] = static_cast<float>(x[i * kP + j]);
    }
    return;
  }
  // panel block: P = A[r0.., kb] L_kk^-T, 64 x 64 x 64 in float64 MFMA (4 x 4 tiles of 16, 4 per wave)
  const int64_t r0 = o + int64_t(blockIdx.x) * kB;
  __syncthreads();
  for (int e = tid; e < kB * kB; e += 256) {  // reuse l for the panel block
    const int i = e >> 6, j = e & 63;
    l[i * kP + j] = static_cast<double>(a[(r0 + i) * dp + o + j]);
  }
  __syncthreads();
  f64x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ti = wave, tj = q;
    f64x4 c = f64x4{};
    for (int u = 0; u <= tj; ++u)  // (L_kk^-T)[u][tj] = M[tj][u], zero for u > tj
      c = mm16<true>(l + 16 * ti * kP + 16 * u, x + 16 * tj * kP + 16 * u, c);
    acc[q] = c;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = 16 * wave + 4 * w + (lane >> 4), j = 16 * q + (lane & 15);
      a[(r0 + i) * dp + o + j] = static_cast<float>(acc[q][w]);
    }
  }
}

// A[i, j] -= L[i, kb] L[j, kb]^T for kb < j <= i.
__global__ __launch_bounds__(256) void update_kernel(float* __restrict__ a, int64_t dp, int kb,
                                                     const int32_t* __restrict__ info) {
  if (*info) return;
  int I, J;
  tri(blockIdx.x, I, J);
  const int64_t o = int64_t(kb) * kB;
  const int64_t ri = o + kB + int64_t(I) * kB, rj = o + kB + int64_t(J) * kB;
  gemm_tile<false, true>(a + ri * dp + o, dp, a + rj * dp + o, dp, a + ri * dp + rj, dp, kB, kB, 0, kB, -1.0f,
                         1.0f);
}

// Merge level with block size s: pair p joins B1 = [2ps, 2ps+s) and B2 = [2ps+s, min(2ps+2s, dp)).
// stage 0: T[B2, B1] = L[B2, B1] M[B1, B1]      (M11 lower: k >= column tile start)
// stage 1: M[B2, B1] = -M[B2, B2] T[B2, B1]     (M22 lower: k <= row tile end)
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ a, float* __restrict__ m,
                                                    float* __restrict__ t, int64_t dp, int64_t s, int tiles_side,
                                                    int stage, const int32_t* __restrict__ info) {
  if (*info) return;
  const int tiles_pair = tiles_side * tiles_side;
  const int64_t p = blockIdx.x / tiles_pair;
  const int tp = blockIdx.x % tiles_pair;
  const int ti = tp / tiles_side, tj = tp % tiles_side;
  const int64_t b1 = 2 * p * s, b2 = b1 + s;
  if (b2 >= dp) return;
  const int64_t n2 = (b2 + s <= dp) ? s : dp - b2;
  const int64_t i0 = int64_t(ti) * kB, j0 = int64_t(tj) * kB;
  if (i0 >= n2) return;
  const int mv = static_cast<int>(n2 - i0 < kB ? n2 - i0 : kB);
  if (stage == 0) {
    // rows of B2, columns of B1, k over B1 from j0
    gemm_tile<false, false>(a + (b2 + i0) * dp + b1, dp, m + b1 * dp + b1 + j0, dp, t + (b2 + i0) * dp + b1 + j0,
                            dp, mv, kB, static_cast<int>(j0), static_cast<int>(s), 1.0f, 0.0f);
  } else {
    const int kend = static_cast<int>(i0 + kB < n2 ? i0 + kB : n2);
    gemm_tile<false, false>(m + (b2 + i0) * dp + b2, dp, t + b2 * dp + b1 + j0, dp, m + (b2 + i0) * dp + b1 + j0,
                            dp, mv, kB, 0, kend, -1.0f, 0.0f);
  }
}

// R[i][j] = M[d-1-i][d-1-j] for i <= j, 0 below the diagonal.
__global__ void output_kernel(const float* __restrict__ m, int64_t d, int64_t dp, float* __restrict__ h) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t i = blockIdx.y;
  if (j >= d) return;
  h[i * d + j] = (i <= j) ? m[(d - 1 - i) * dp + (d - 1 - j)] : 0.0f;
}

struct Layout {
  int64_t dp;
  size_t a_off, m_off, t_off, delta_off, total;
};

Layout layout(int64_t d) {
  Layout l{};
  l.dp = (d + kB - 1) / kB * kB;
  const size_t mat = align_up(size_t(l.dp) * l.dp * sizeof(float), 256);
  l.a_off = 0;
  l.m_off = mat;
  l.t_off = 2 * mat;
  l.delta_off = 3 * mat;
  l.total = 3 * mat + 256;
  return l;
}

}  // namespace

size_t chol_workspace(int64_t d) { return layout(d).total; }

kq_status chol_run(float* h, int64_t d, float damp, int32_t* info, void* ws, hipStream_t st) {
  const Layout L = layout(d);
  char* base = static_cast<char*>(ws);
  float* a = reinterpret_cast<float*>(base + L.a_off);
  float* m = reinterpret_cast<float*>(base + L.m_off);
  float* t = reinterpret_cast<float*>(base + L.t_off);
  double* delta = reinterpret_cast<double*>(base + L.delta_off);
  const int64_t dp = L.dp;
  const int nb = static_cast<int>(dp / kB);
  kq_status r;

  {
    LaunchTimer timer("damp_kernel", st);
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, st, h, d, damp, delta, info);
  }
  if ((r = check_launch("damp_kernel")) != KQ_OK) return r;
  // M is never read above its diagonal 64 x 64 blocks, so it needs no clearing.
  {
    LaunchTimer timer("reverse_kernel", st);
    hipLaunchKernelGGL(reverse_kernel, dim3(static_cast<unsigned>((dp + 255) / 256), static_cast<unsigned>(dp)),
                       dim3(256), 0, st, h, d, dp, delta, a);
  }
  if ((r = check_launch("reverse_kernel")) != KQ_OK) return r;

  for (int kb = 0; kb < nb; ++kb) {
    const int rest = nb - kb - 1;
    {
      LaunchTimer timer("diag_panel_kernel", st);
      hipLaunchKernelGGL(diag_panel_kernel, dim3(static_cast<unsigned>(1 + rest)), dim3(256), 0, st, a, m, dp, kb,
                         d, info);
    }
    if ((r = check_launch("diag_panel_kernel")) != KQ_OK) return r;
    if (rest == 0) break;
    {
      LaunchTimer timer("update_kernel", st);
      hipLaunchKernelGGL(update_kernel, dim3(static_cast<unsigned>(rest * (rest + 1) / 2)), dim3(256), 0, st, a, dp,
                         kb, info);
    }
    if ((r = check_launch("update_kernel")) != KQ_OK) return r;
  }

  for (int64_t s = kB; s < dp; s *= 2) {
    const int64_t pairs = (dp + 2 * s - 1) / (2 * s);
    const int tiles_side = static_cast<int>(s / kB);
    const unsigned grid = static_cast<unsigned>(pairs * tiles_side * tiles_side);
    for (int stage = 0; stage < 2; ++stage) {
      {
        LaunchTimer timer("merge_kernel", st);
        hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(256), 0, st, a, m, t, dp, s, tiles_side, stage, info);
      }
      if ((r = check_launch("merge_kernel")) != KQ_OK) return r;
    }
  }

  {
    LaunchTimer timer("output_kernel", st);
    hipLaunchKernelGGL(output_kernel, dim3(static_cast<unsigned>((d + 255) / 256), static_cast<unsigned>(d)),
                       dim3(256), 0, st, m, d, dp, h);
  }
  return check_launch("output_kernel");
}

}  // namespace kq
