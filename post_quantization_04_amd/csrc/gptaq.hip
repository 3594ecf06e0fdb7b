// Row f2, the GPTAQ base quantizer: drift-corrected weights before GPTQ's sweep.
//
// KronQ's column update is GPTAQ's, which corrects GPTQ for the drift between
// the inputs the partly quantized model feeds a layer and those of the
// full-precision model (wmrh.cn KronQ article, sections 四 and 八; the pages
// give no formula). Reading implemented: with X the quantized-model inputs,
// dX the drift, D = dX^T X / N and R upper with R^T R = H~^-1 (the damped
// H_X's factor, as the sweep uses it), each column q's drift w_q dx_q is
// compensated by least squares on the later columns' inputs, which moves the
// later columns by w_q D_{q,>q} H~_{>q,>q}^-1; the trailing block's inverse is
// R_{>q,>q}^T R_{>q,>q}, so all compensations together are
//     W' = W + W P,   P = triu(D R^T, 1) R,
// and GPTQ's sweep then runs on W'. Everything here is in the basis of the
// sweep (after BiIP: D'' and R of H_X'').
//
// Three float64 products on v_mfma_f64_16x16x4f64, 64 x 64 output tiles
// (4 waves of 32 x 32), k in chunks of 16 through LDS, with the triangles
// skipped:
//   1. Y = triu(D R^T, 1):  Y[q][k] = sum_{j >= k} D[q][j] R[k][j], k > q;
//   2. Z = W Y:             Z[i][k] = sum_{q < k} W[i][q] Y[q][k];
//   3. W += Z R:            W[i][j] += sum_{k <= j} Z[i][k] R[k][j].
// Every sum runs in a fixed order, so results repeat bit for bit.
#include "kq_internal.h"

namespace kq {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 64;       // output tile edge
constexpr int kK = 16;       // k chunk
constexpr int kPad = kT + 2; // LDS row pitch (doubles)

struct TileLds {
  double a[2][kK][kPad];  // [k][row]
  double b[2][kK][kPad];  // [k][column]
};

// k range of an output tile with first column j0: K_FROM_COL sums k in [j0, K)
// (B(k, j) = 0 for k < j), K_TO_COL sums k in [0, j0 + 64) (B(k, j) = 0 for k > j).
enum KRange { K_FROM_COL = 0, K_TO_COL = 1 };

// out[i][j] = (ACC ? out[i][j] : 0) + sum_k A(i, k) B(k, j) over the tile's k range, with
// A(i, k) = a[i * lda + k] and B(k, j) = TRANSB ? b[j * ldb + k] : b[k * ldb + j]. MASK keeps
// the strict upper triangle (j > i) and writes zeros elsewhere; tiles wholly on or below the
// diagonal skip the products. Entries past M, N or the k range read as zero.
template <typename TA, typename TB, bool TRANSB, int KR, bool ACC, bool MASK>
__global__ __launch_bounds__(256) void gemm_kernel(const TA* __restrict__ a, int64_t lda, const TB* __restrict__ b,
                                                   int64_t ldb, double* __restrict__ out, int64_t ldo, int64_t M,
                                                   int64_t N, int64_t K, int64_t tiles_j) {
  __shared__ TileLds sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t t = blockIdx.x;
  const int64_t i0 = (t / tiles_j) * kT, j0 = (t % tiles_j) * kT;
  // D[i][j] of a 16 x 16 float64 block: lane l, register q -> i = 4 q + l / 16, j = l % 16
  const int il = lane & 15, kl = lane >> 4;
  auto store_out = [&](const f64x4 (&acc)[2][2]) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t i = i0 + wi * 32 + x * 16 + 4 * q + kl, j = j0 + wj * 32 + y * 16 + il;
          if (i >= M || j >= N) continue;
          double v = acc[x][y][q];
          if (MASK && j <= i) v = 0.0;
          if (ACC) v += out[i * ldo + j];
          out[i * ldo + j] = v;
        }
  };
  f64x4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{};
  if (MASK && j0 + kT - 1 <= i0) {  // every entry of the tile has j <= i
    store_out(acc);
    return;
  }
  const int64_t klo = KR == K_FROM_COL ? j0 : 0;
  const int64_t khi = KR == K_FROM_COL ? K : (j0 + kT < K ? j0 + kT : K);
  // one chunk: 64 x 16 of A and 16 x 64 of B, 4 elements of each per thread
  double va[4], vb[4];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      const int ar = e >> 4, ak = e & 15;  // A: row ar, k ak (rows contiguous in k)
      const int64_t gi = i0 + ar, gk = k0 + ak;
      va[u] = (gi < M && gk < khi) ? static_cast<double>(a[gi * lda + gk]) : 0.0;
      if (TRANSB) {
        const int bj = e >> 4, bk = e & 15;  // B^T rows contiguous in k
        const int64_t gj = j0 + bj, gk2 = k0 + bk;
        vb[u] = (gj < N && gk2 < khi) ? static_cast<double>(b[gj * ldb + gk2]) : 0.0;
      } else {
        const int bk = e >> 6, bj = e & 63;  // B rows contiguous in j
        const int64_t gk2 = k0 + bk, gj = j0 + bj;
        vb[u] = (gk2 < khi && gj < N) ? static_cast<double>(b[gk2 * ldb + gj]) : 0.0;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      sm.a[buf][e & 15][e >> 4] = va[u];
      if (TRANSB) sm.b[buf][e & 15][e >> 4] = vb[u];
      else sm.b[buf][e >> 6][e & 63] = vb[u];
    }
  };
  const int64_t nch = khi > klo ? (khi - klo + kK - 1) / kK : 0;
  if (nch > 0) {
    load(klo);
    store(0);
  }
  __syncthreads();
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int buf = static_cast<int>(ch & 1);
    if (ch + 1 < nch) load(klo + (ch + 1) * kK);
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
  store_out(acc);
}

template <typename TA, typename TB, bool TRANSB, int KR, bool ACC, bool MASK>
kq_status gemm(const char* name, const TA* a, int64_t lda, const TB* b, int64_t ldb, double* out, int64_t ldo,
               int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t ti = (M + kT - 1) / kT, tj = (N + kT - 1) / kT;
  if (ti * tj == 0) return KQ_OK;
  {
    LaunchTimer timer(name, st);
    hipLaunchKernelGGL((gemm_kernel<TA, TB, TRANSB, KR, ACC, MASK>), dim3(static_cast<unsigned>(ti * tj)), dim3(256),
                       0, st, a, lda, b, ldb, out, ldo, M, N, K, tj);
  }
  return check_launch(name);
}

struct Layout {
  size_t y_bytes, z_bytes;
};

Layout layout(int64_t dout, int64_t din) {
  return Layout{align_up(size_t(din) * din * sizeof(double), 256), align_up(size_t(dout) * din * sizeof(double), 256)};
}

}  // namespace

size_t gptaq_workspace(int64_t dout, int64_t din) {
  const Layout l = layout(dout, din);
  return l.y_bytes + l.z_bytes;
}

kq_status gptaq_target_run(double* w, const float* d2, const float* r, int64_t dout, int64_t din, void* ws,
                           hipStream_t st) {
  const Layout l = layout(dout, din);
  double* y = static_cast<double*>(ws);
  double* z = reinterpret_cast<double*>(static_cast<char*>(ws) + l.y_bytes);
  // 1. Y = triu(D R^T, 1): B(j, k) = R[k][j]
  kq_status s = gemm<float, float, true, K_FROM_COL, false, true>("gptaq_drift_kernel", d2, din, r, din, y, din, din,
                                                                  din, din, st);
  if (s != KQ_OK) return s;
  // 2. Z = W Y
  s = gemm<double, double, false, K_TO_COL, false, false>("gptaq_weight_kernel", w, din, y, din, z, din, dout, din,
                                                          din, st);
  if (s != KQ_OK) return s;
  // 3. W += Z R
  return gemm<double, float, false, K_TO_COL, true, false>("gptaq_update_kernel", z, din, r, din, w, din, dout, din,
                                                           din, st);
}

}  // namespace kq
