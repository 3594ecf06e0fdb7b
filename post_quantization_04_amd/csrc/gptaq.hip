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
// Three float64 products on v_mfma_f64_16x16x4f64, 128 x 128 output tiles
// (4 waves of 64 x 64), k in chunks of 16 through LDS, with the triangles
// skipped:
//   1. Y = triu(D R^T, 1):  Y[q][k] = sum_{j >= k} D[q][j] R[k][j], k > q;
//   2. Z = W Y:             Z[i][k] = sum_{q < k} W[i][q] Y[q][k];
//   3. W += Z R:            W[i][j] += sum_{k <= j} Z[i][k] R[k][j].
// Every sum runs in a fixed order, so results repeat bit for bit.
#include "kq_internal.h"

namespace kq {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 128;       // output tile edge (4 waves of 64 x 64)
constexpr int kK = 16;        // k chunk
constexpr int kRowPitch = kK + 2;  // LDS pitch of a [row][k] panel (doubles)
constexpr int kColPitch = kT + 16; // LDS pitch of a [k][column] panel (doubles)
constexpr int kMaxSuper = 8;  // super-tiles of up to 8 x 8 tiles, each run by one XCD
constexpr int kXcds = 8;

// k range of an output tile with first column j0: K_FROM_COL sums k in [j0, K)
// (B(k, j) = 0 for k < j), K_TO_COL sums k in [0, j0 + 128) (B(k, j) = 0 for k > j).
enum KRange { K_FROM_COL = 0, K_TO_COL = 1 };

template <bool TRANSB>
struct TileLds {
  double a[2][kT][kRowPitch];                                   // [row][k]
  double b[2][TRANSB ? kT : kK][TRANSB ? kRowPitch : kColPitch];  // [column][k] or [k][column]
};

// out[i][j] = (ACC ? out[i][j] : 0) + sum_k A(i, k) B(k, j) over the tile's k range, with
// A(i, k) = a[i * lda + k] and B(k, j) = TRANSB ? b[j * ldb + k] : b[k * ldb + j]. MASK keeps
// the strict upper triangle (j > i) of the tiles on or above the diagonal, with zeros at j <= i
// inside them, and leaves the tiles wholly below the diagonal unwritten (a product with the
// result, over the k range of K_TO_COL, reads only the tiles on or above it). Entries past the
// k range count as zero.
//
// Float64 MFMA issues one 16 x 16 x 4 product per 64 cycles on a SIMD, so a 128 x 128 tile
// needs 32 KB of operands per 4096 cycles of a wave's MFMA work. Workgroups run as sup x sup-tile
// super-tiles (sup = 8 at large sizes), each on one XCD (workgroups are dispatched to the XCDs
// in turn): the tiles running together there share sup row panels of A and sup column panels
// of B through that XCD's L2. The super-tiles that hold work are numbered column by column in
// order of falling k range (the longest tiles start first) and dealt to the XCDs in turn, so
// each XCD gets an even share of the work; with MASK only those on or above the diagonal.
template <typename TA, typename TB, bool TRANSB, int KR, bool ACC, bool MASK, bool CHECK>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const TA* __restrict__ a, int64_t lda,
                                                      const TB* __restrict__ b, int64_t ldb,
                                                      double* __restrict__ out, int64_t ldo, int64_t M,
                                                      int64_t N, int64_t K, int sup, int super_i, int super_j,
                                                      int n_super, int32_t* __restrict__ info) {
  __shared__ TileLds<TRANSB> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  int s = (local / (sup * sup)) * kXcds + xcd;
  const int within = local % (sup * sup);
  if (s >= n_super) return;
  // super-tile s -> (si, sj): columns in order of falling k range, super_i entries each (MASK:
  // the min(sj + 1, super_i) on or above the diagonal)
  int sj_ord = 0;
  if constexpr (MASK) {
    for (;;) {
      const int col = KR == K_TO_COL ? super_j - 1 - sj_ord : sj_ord;
      const int c = col + 1 < super_i ? col + 1 : super_i;
      if (s < c) break;
      s -= c;
      ++sj_ord;
    }
  } else {
    sj_ord = s / super_i;
    s -= sj_ord * super_i;
  }
  const int si = s;
  const int sj = KR == K_TO_COL ? super_j - 1 - sj_ord : sj_ord;
  const int64_t ti = int64_t(si) * sup + within / sup, tj = int64_t(sj) * sup + within % sup;
  const int64_t i0 = ti * kT, j0 = tj * kT;
  if (i0 >= M || j0 >= N) return;
  if (MASK && tj < ti) return;  // wholly below the diagonal: not written
  // D[i][j] of a 16 x 16 float64 block: lane l, register q -> i = 4 q + l / 16, j = l % 16
  const int il = lane & 15, kl = lane >> 4;
  f64x4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f64x4{};
  const int64_t klo = KR == K_FROM_COL ? j0 : 0;
  const int64_t khi = KR == K_FROM_COL ? K : (j0 + kT < K ? j0 + kT : K);
  const int64_t nch = khi > klo ? (khi - klo + kK - 1) / kK : 0;
  // one chunk: 128 x 16 of A and 16 x 128 of B, 8 elements of each per thread, in pairs along
  // the contiguous index (rows of A and of B^T in k, rows of B in j). They stay as loaded until
  // the LDS store, so the next chunk's loads are in flight during the current chunk's products.
  // Indices are clamped so every load reads valid memory: a row of A past M or a column of B
  // past N feeds only outputs that are not written, and entries at k >= khi are stored as zero.
  const int kp = (tid & 7) * 2;            // A and B^T: k pair of this thread
  const int kr0 = tid >> 6, jp = (tid & 63) * 2;  // B: k row (+ 4 u) and column pair
  const TA* arow[4];
  const TB* bcol[4];  // TRANSB: rows of B^T
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t gi = i0 + (tid >> 3) + 32 * u;
    arow[u] = a + (gi < M ? gi : M - 1) * lda;
    if constexpr (TRANSB) {
      const int64_t gj = j0 + (tid >> 3) + 32 * u;
      bcol[u] = b + (gj < N ? gj : N - 1) * ldb;
    }
  }
  const int64_t gj0 = j0 + jp < N ? j0 + jp : N - 1, gj1 = j0 + jp + 1 < N ? j0 + jp + 1 : N - 1;
  TA va[8];
  TB vb[8];
  auto load = [&](int64_t k0) {
    const int64_t k_0 = k0 + kp < K ? k0 + kp : K - 1, k_1 = k0 + kp + 1 < K ? k0 + kp + 1 : K - 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      va[2 * u] = arow[u][k_0];
      va[2 * u + 1] = arow[u][k_1];
      if constexpr (TRANSB) {
        vb[2 * u] = bcol[u][k_0];
        vb[2 * u + 1] = bcol[u][k_1];
      } else {
        const int64_t gk = k0 + kr0 + 4 * u < K ? k0 + kr0 + 4 * u : K - 1;
        vb[2 * u] = b[gk * ldb + gj0];
        vb[2 * u + 1] = b[gk * ldb + gj1];
      }
    }
  };
  auto store = [&](int buf, int64_t k0) {
    const int64_t kmax = khi - k0;  // chunk entries at k >= kmax are zero
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (tid >> 3) + 32 * u;
      sm.a[buf][r][kp] = kp < kmax ? static_cast<double>(va[2 * u]) : 0.0;
      sm.a[buf][r][kp + 1] = kp + 1 < kmax ? static_cast<double>(va[2 * u + 1]) : 0.0;
      if constexpr (TRANSB) {
        sm.b[buf][r][kp] = kp < kmax ? static_cast<double>(vb[2 * u]) : 0.0;
        sm.b[buf][r][kp + 1] = kp + 1 < kmax ? static_cast<double>(vb[2 * u + 1]) : 0.0;
      } else {
        const int kr = kr0 + 4 * u;
        sm.b[buf][kr][jp] = kr < kmax ? static_cast<double>(vb[2 * u]) : 0.0;
        sm.b[buf][kr][jp + 1] = kr < kmax ? static_cast<double>(vb[2 * u + 1]) : 0.0;
      }
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kK / 4; ++kk) {
      const int kr = 4 * kk + kl;
      double fa[4], fb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) fa[x] = sm.a[buf][wi * 64 + x * 16 + il][kr];
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        if constexpr (TRANSB) fb[y] = sm.b[buf][wj * 64 + y * 16 + il][kr];
        else fb[y] = sm.b[buf][kr][wj * 64 + y * 16 + il];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
  };
  if (nch > 0) {
    load(klo);
    store(0, klo);
  }
  __syncthreads();
  // every chunk but the last: next chunk's loads, this chunk's products, next chunk's store
  for (int64_t ch = 0; ch + 1 < nch; ++ch) {
    const int64_t k1 = klo + (ch + 1) * kK;
    load(k1);
    mma(static_cast<int>(ch & 1));
    store(static_cast<int>((ch + 1) & 1), k1);
    __syncthreads();
  }
  if (nch > 0) mma(static_cast<int>((nch - 1) & 1));
  bool bad = false;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t i = i0 + wi * 64 + x * 16 + 4 * q + kl, j = j0 + wj * 64 + y * 16 + il;
        if (i >= M || j >= N) continue;
        double v = acc[x][y][q];
        if (MASK && j <= i) v = 0.0;
        if (ACC) v += out[i * ldo + j];
        out[i * ldo + j] = v;
        if (CHECK) bad = bad || !isfinite(v);
      }
  if (CHECK && bad && info) atomicOr(info, 1);
}

template <typename TA, typename TB, bool TRANSB, int KR, bool ACC, bool MASK, bool CHECK = false>
kq_status gemm(const char* name, const TA* a, int64_t lda, const TB* b, int64_t ldb, double* out, int64_t ldo,
               int64_t M, int64_t N, int64_t K, hipStream_t st, int32_t* info = nullptr) {
  const int64_t ti = (M + kT - 1) / kT, tj = (N + kT - 1) / kT;
  if (ti * tj == 0) return KQ_OK;
  // the largest super-tile edge that still deals at least 16 super-tiles with work to each XCD
  // (smaller edges share less through L2 but balance short launches better)
  int sup = kMaxSuper;
  int64_t super_i = 0, super_j = 0, n_super = 0;
  for (;; sup /= 2) {
    super_i = (ti + sup - 1) / sup;
    super_j = (tj + sup - 1) / sup;
    n_super = 0;
    if (MASK) {
      for (int64_t c = 0; c < super_j; ++c) n_super += c + 1 < super_i ? c + 1 : super_i;
    } else {
      n_super = super_i * super_j;
    }
    if (sup == 1 || n_super >= 16 * kXcds) break;
  }
  // every XCD runs the same number of super-tile slots (the surplus workgroups return at once)
  const int64_t rounds = (n_super + kXcds - 1) / kXcds;
  const int64_t blocks = rounds * kXcds * sup * sup;
  if (blocks > INT32_MAX) return fail(KQ_EUNSUPPORTED, "%s: %lld x %lld output too large", name, (long long)M,
                                      (long long)N);
  {
    LaunchTimer timer(name, st);
    hipLaunchKernelGGL((gemm_kernel<TA, TB, TRANSB, KR, ACC, MASK, CHECK>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, st, a, lda, b, ldb, out, ldo, M, N, K, sup, static_cast<int>(super_i),
                       static_cast<int>(super_j), static_cast<int>(n_super), info);
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

kq_status gptaq_target_run(double* w, const float* d2, const float* r, int64_t dout, int64_t din, int32_t* info,
                           void* ws, hipStream_t st) {
  const Layout l = layout(dout, din);
  double* y = static_cast<double*>(ws);
  double* z = reinterpret_cast<double*>(static_cast<char*>(ws) + l.y_bytes);
  // 1. Y = triu(D R^T, 1): B(j, k) = R[k][j]; the tiles of Y below the diagonal stay unwritten (the
  //    next product's k range stops at the diagonal tile)
  kq_status s = gemm<float, float, true, K_FROM_COL, false, true>("gptaq_drift_kernel", d2, din, r, din, y, din, din,
                                                                  din, din, st);
  if (s != KQ_OK) return s;
  // 2. Z = W Y
  s = gemm<double, double, false, K_TO_COL, false, false>("gptaq_weight_kernel", w, din, y, din, z, din, dout, din,
                                                          din, st);
  if (s != KQ_OK) return s;
  // 3. W += Z R; a corrected weight that is not finite sets *info
  return gemm<double, float, false, K_TO_COL, true, false, true>("gptaq_update_kernel", z, din, r, din, w, din, dout,
                                                                 din, din, st, info);
}

}  // namespace kq
