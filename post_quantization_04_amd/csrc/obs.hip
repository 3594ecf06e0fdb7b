// GPTQ-style column-wise OBS on the rotated weight, in float64.
//
// The sweep is sequential in the column index and independent across rows,
// given R. Per block k of B columns [c0, c0 + B), one launch with two roles:
//     - sweep (16 rows per workgroup): 16 lanes own one row; lane l keeps
//       columns l, l + 16, ... of the block in registers (B / 16 values).
//       First (k > 0) the registers receive the previous block's errors of
//       the same rows, W[r, c0:c0+B] -= E_{k-1}[r] R[c0-B:c0, c0:c0+B], one
//       16-row product on float64 MFMA; the workgroup wrote those errors
//       itself one launch earlier. For
//       column j the owning lane quantises, forms the scaled error
//       e = (w - w^) / R_jj and the error is broadcast to the row's 16 lanes
//       with one DPP row_newbcast; every lane then removes e * R[j][k] from
//       its columns k. The block of R sits in LDS, laid out so each lane reads
//       its B / 16 entries of row j; entries on and below the diagonal are
//       stored as zero, so the update is branch free. Group minima and maxima
//       are 16-lane shuffle reductions. The block's errors go to E_k.
//     - far update (lazy batch): W[:, c0+B:] -= E_{k-1} R[c0-B:c0, c0+B:] on
//       float64 MFMA (v_mfma_f64_16x16x4f64) in 128 x 128 tiles.
//     The roles touch disjoint columns and E is double buffered, so the
//     latency-bound sweep (one wave per SIMD) shares the GPU with the
//     MFMA-bound update instead of alternating with it.
// Float64 keeps the rounding argument w / s of every entry within about
// 1e-6 grid units of the float64 oracle across thousands of columns, where a
// float32 sweep drifts past 1e-5.
#include <type_traits>

#include "kq_internal.h"

namespace kq {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kSweepThreads = 256;  // 16 rows per workgroup
constexpr int kRowsPerWg = kSweepThreads / 16;

template <int CTRL>
__device__ __forceinline__ double dpp_bcast(double v) {
  // every lane reads a valid source under row_newbcast, so no "old" value is needed
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

// Value of lane `src` of this lane's group of 16 (row_newbcast), src uniform.
__device__ __forceinline__ double bcast16(double v, int src) {
  switch (src) {
    case 0: return dpp_bcast<0x150>(v);
    case 1: return dpp_bcast<0x151>(v);
    case 2: return dpp_bcast<0x152>(v);
    case 3: return dpp_bcast<0x153>(v);
    case 4: return dpp_bcast<0x154>(v);
    case 5: return dpp_bcast<0x155>(v);
    case 6: return dpp_bcast<0x156>(v);
    case 7: return dpp_bcast<0x157>(v);
    case 8: return dpp_bcast<0x158>(v);
    case 9: return dpp_bcast<0x159>(v);
    case 10: return dpp_bcast<0x15A>(v);
    case 11: return dpp_bcast<0x15B>(v);
    case 12: return dpp_bcast<0x15C>(v);
    case 13: return dpp_bcast<0x15D>(v);
    case 14: return dpp_bcast<0x15E>(v);
    default: return dpp_bcast<0x15F>(v);
  }
}

// Asymmetric min-max grid; the scale is rounded to float32 (its stored form).
__device__ __forceinline__ void make_grid(double mn, double mx, int maxq, double& s, double& z) {
  double xmin = fmin(mn, 0.0), xmax = fmax(mx, 0.0);
  if (xmin == 0.0 && xmax == 0.0) {
    xmin = -1.0;
    xmax = 1.0;
  }
  s = static_cast<double>(static_cast<float>((xmax - xmin) / static_cast<double>(maxq)));
  z = fmin(fmax(rint(-xmin / s), 0.0), static_cast<double>(maxq));
}

// One grid per row (group == 0), from the weights before the sweep. One wave per row.
__global__ __launch_bounds__(256) void row_grid_kernel(const double* __restrict__ w, int64_t dout, int64_t din,
                                                       int bits, float* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= dout) return;
  const int lane = threadIdx.x & 63;
  double mn = INFINITY, mx = -INFINITY;
  for (int64_t j = lane; j < din; j += 64) {
    const double v = w[row * din + j];
    mn = fmin(mn, v);
    mx = fmax(mx, v);
  }
  for (int o = 32; o > 0; o >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, o, 64));
    mx = fmax(mx, __shfl_xor(mx, o, 64));
  }
  if (lane == 0) {
    double s, z;
    make_grid(mn, mx, (1 << bits) - 1, s, z);
    scales[row] = static_cast<float>(s);
    zeros[row] = static_cast<uint8_t>(z);
  }
}

// Shared memory of the sweep: rl[j][l * EPL + e] = R[c0 + j][c0 + l + 16 e]
// above the diagonal, else 0; rinv[j] = 1 / R[c0 + j][c0 + j].
template <int B>
struct SweepLds {
  float rl[B][B];
  double rinv[B];
};

// Group start at column j of the block: grid of columns [j, j + group) from
// this row's current values (16-lane min / max reduction), stored by lane 0.
template <int EPL>
__device__ __forceinline__ void group_start(const double (&x)[EPL], int eo, int j, int l16, int group, int log2g,
                                            int maxq, bool valid, int64_t row, int64_t ngroups, int64_t c0,
                                            float* __restrict__ scales, uint8_t* __restrict__ zeros, double& s,
                                            double& z, double& inv_s) {
  double mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int col = l16 + 16 * (eo + e);
    if (col >= j && col < j + group) {
      mn = fmin(mn, x[e]);
      mx = fmax(mx, x[e]);
    }
  }
  for (int o = 8; o > 0; o >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, o, 16));
    mx = fmax(mx, __shfl_xor(mx, o, 16));
  }
  make_grid(mn, mx, maxq, s, z);
  inv_s = 1.0 / s;
  if (l16 == 0 && valid) {
    const int64_t gi = row * ngroups + ((c0 + j) >> log2g);
    scales[gi] = static_cast<float>(s);
    zeros[gi] = static_cast<uint8_t>(z);
  }
}

// A B x B block of R in registers: this thread's 16-byte pieces of it.
template <int B>
struct RBlock {
  static constexpr int V = B / 4, N = B * V / kSweepThreads;
  static_assert(N >= 1 && B * V % kSweepThreads == 0, "block shape");
  float4 v[N];
};

// Issues the loads of R[row0 .. row0 + B, col0 .. col0 + B] into rb.
template <int B>
__device__ __forceinline__ void load_r(RBlock<B>& rb, const float* __restrict__ r, int64_t din, int64_t row0,
                                       int64_t col0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < RBlock<B>::N; ++q) {
    const int idx = tid + q * kSweepThreads, j = idx / RBlock<B>::V, k4 = (idx % RBlock<B>::V) * 4;
    rb.v[q] = *reinterpret_cast<const float4*>(r + (row0 + j) * din + col0 + k4);
  }
}

// rl[j][l * EPL + e] = R[row0 + j][col0 + l + 16 e] for the block in rb (upper: entries on
// and below the diagonal stored as 0).
template <int B, bool UPPER>
__device__ __forceinline__ void store_r(const RBlock<B>& rb, float (&rl)[B][B]) {
  constexpr int EPL = B / 16;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < RBlock<B>::N; ++q) {
    const int idx = tid + q * kSweepThreads, j = idx / RBlock<B>::V, k4 = (idx % RBlock<B>::V) * 4;
    const float f[4] = {rb.v[q].x, rb.v[q].y, rb.v[q].z, rb.v[q].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int k = k4 + t;
      rl[j][(k & 15) * EPL + (k >> 4)] = (!UPPER || k > j) ? f[t] : 0.0f;
    }
  }
}

// Workgroup barrier that waits for this wave's LDS accesses only: global loads
// issued before it stay in flight (__syncthreads would wait for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Sweep of block [c0, c0 + B) for rows [16 wg, 16 wg + 16). First the errors of
// the nq blocks before it that no earlier launch applied to it (nq = 1 inside a
// super-block, kSB at its first block) are applied: e_prev holds them for
// columns c0 - nq B .. c0, rows of pitch pe. Then the sweep; the block's scaled
// errors go to e_out (rows of pitch pe). Groups are powers of two dividing B:
// with SG false (no group, or group >= 16) a group can start only at a
// 16-column slice, so the grid code sits outside the unrolled column loop.
template <int B, bool SG, bool TL>
__device__ void sweep_role(SweepLds<B>& sm, int wg, double* __restrict__ w, const float* __restrict__ r,
                           int64_t dout, int64_t din, int64_t c0, int bits, int group, uint8_t* __restrict__ codes,
                           float* __restrict__ scales, uint8_t* __restrict__ zeros, double* __restrict__ preround,
                           const double* __restrict__ e_prev, int nq, double* __restrict__ e_out, int pe) {
  constexpr int EPL = B / 16;
  auto& rl = sm.rl;
  auto& rinv = sm.rinv;
  const int tid = threadIdx.x;
  const int l16 = tid & 15;
  const int64_t row = int64_t(wg) * kRowsPerWg + (tid >> 4);
  const bool valid = row < dout;
  const int maxq = (1 << bits) - 1;
  const int64_t ngroups = group ? din / group : 1;
  const int gmask = group - 1;
  const int log2g = group ? __builtin_ctz(static_cast<unsigned>(group)) : 0;

  // x[e] holds column l16 + 16 (eo + e) of this lane's row: the slice being
  // swept is always x[0]; registers rotate down after each slice of 16 columns.
  double x[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = valid ? w[row * din + c0 + l16 + 16 * e] : 0.0;
  // the block's own R block is loaded now and staged after the previous block's update,
  // so its loads overlap that update
  RBlock<B> rdiag;
  // 1 / R_jj of the block, one division per thread j < B
  const float rjj = tid < B ? r[(c0 + tid) * din + c0 + tid] : 1.0f;
  if (c0 > 0) {
    // earlier blocks' errors of these rows: x -= E_prev R[c0-nq B:c0, c0:c0+B] for the
    // workgroup's 16 rows, as a 16 x (nq B) x B product on float64 MFMA (v_mfma_f64_16x16x4f64),
    // one B x B block of R at a time, staged in the sweep's LDS layout (all entries)
    constexpr int KS = B / 4, NT = B / 16, TPW = (NT + 3) / 4;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t erow = int64_t(wg) * kRowsPerWg + (lane & 15);
    f64x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = f64x4{};
    const int nqb = TL ? nq : 1;  // one-level: always the previous block only
    // one earlier block q of R; the last one also loads the block's own R (peeled, so that
    // block is live only there and the runtime loop over the others holds one R block)
    auto near = [&](int q, auto last) {
      RBlock<B> rnear;
      load_r<B>(rnear, r, din, c0 - int64_t(nqb - q) * B, c0);
      if constexpr (decltype(last)::value) load_r<B>(rdiag, r, din, c0, c0);
      // A operand of k-step kk: lane i + 16 c holds E_prev[row i of the workgroup][q B + 4 kk + c]
      const double* ep = e_prev + (erow < dout ? erow : 0) * pe + q * B + (lane >> 4);
      double ea[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) ea[kk] = ep[4 * kk];
      if (q > 0) lds_barrier();  // every wave is done reading the previous R block
      store_r<B, false>(rnear, rl);
      lds_barrier();
      // 16-column tiles: wave w takes tiles w, w + 4, ...; B operand of k-step kk for tile t:
      // lane j + 16 c holds R[c0 - (nq - q) B + 4 kk + c][c0 + 16 t + j] = rl[4 kk + c][j EPL + t]
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const int t = wave + 4 * u;
          if (t < NT)
            acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                ea[kk], static_cast<double>(rl[4 * kk + (lane >> 4)][(lane & 15) * EPL + t]), acc[u], 0, 0, 0);
        }
    };
    if constexpr (TL)
      for (int q = 0; q + 1 < nqb; ++q) near(q, std::false_type{});
    near(nqb - 1, std::true_type{});
    lds_barrier();  // every wave is done reading the last R block
    // the product, row 4 q + lane / 16 and column 16 t + lane % 16 in register q, goes through
    // LDS (over the R block just read) into the sweep layout
    double (*prod)[B] = reinterpret_cast<double (*)[B]>(&rl[0][0]);
    static_assert(kRowsPerWg * B * sizeof(double) <= sizeof(rl), "product fits over the R block");
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave + 4 * u;
      if (t < NT) {
#pragma unroll
        for (int q = 0; q < 4; ++q) prod[4 * q + (lane >> 4)][16 * t + (lane & 15)] = acc[u][q];
      }
    }
    lds_barrier();
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] -= prod[tid >> 4][l16 + 16 * e];
    lds_barrier();  // the product is read before the block's own R overwrites it
  } else {
    load_r<B>(rdiag, r, din, c0, c0);
  }
  store_r<B, true>(rdiag, rl);
  if (tid < B) rinv[tid] = 1.0 / static_cast<double>(rjj);
  lds_barrier();
  double s = 1.0, z = 0.0;
  if (group == 0 && valid) {
    s = static_cast<double>(scales[row]);
    z = static_cast<double>(zeros[row]);
  }
  double inv_s = 1.0 / s;

  // Fully unrolled: x[e] is column l16 + 16 e throughout. Within slice eo only x[eo] is on
  // the dependent chain (quantise, broadcast, one FMA per column, with the slice's 16 R
  // entries loaded up front); the updates of the later slices x[e > eo] follow as one batch
  // at the end of the slice, in the same per-element order as column by column.
#pragma unroll
  for (int eo = 0; eo < EPL; ++eo) {
    if (!SG && group > 0 && ((eo * 16) & gmask) == 0)
      group_start<EPL>(x, 0, eo * 16, l16, group, log2g, maxq, valid, row, ngroups, c0, scales, zeros, s, z, inv_s);
    const double rcur = rinv[eo * 16 + l16];  // 1 / R_jj of this lane's column of the slice
    float rd[16];                              // R[eo 16 + lo][this lane's column of the slice]
#pragma unroll
    for (int lo = 0; lo < 16; ++lo) rd[lo] = rl[eo * 16 + lo][l16 * EPL + eo];
    double eb[16];
    double tcur = 0.0, ecur = 0.0, qcur = 0.0;
#pragma unroll
    for (int lo = 0; lo < 16; ++lo) {
      const int j = eo * 16 + lo;
      if (SG && (j & gmask) == 0)
        group_start<EPL>(x, 0, j, l16, group, log2g, maxq, valid, row, ngroups, c0, scales, zeros, s, z, inv_s);
      // the rounding argument w * (1/s) is within two ulps of w / s
      const double wv = x[eo];
      const double t = wv * inv_s;
      const double q = fmin(fmax(rint(t) + z, 0.0), static_cast<double>(maxq));
      const double wq = s * (q - z);
      const double err = (wv - wq) * rcur;
      const bool own = l16 == lo;
      tcur = own ? t : tcur;
      ecur = own ? err : ecur;
      qcur = own ? q : qcur;
      eb[lo] = bcast16(err, lo);
      // R[j][own column] and R[j][earlier columns] are stored as 0: those lanes keep their value
      x[eo] = fma(-eb[lo], static_cast<double>(rd[lo]), own ? wq : wv);
    }
    if (valid) {
      const int64_t col = c0 + l16 + 16 * eo;
      w[row * din + col] = x[eo];
      codes[row * din + col] = static_cast<uint8_t>(qcur);
      if (preround) preround[row * din + col] = tcur;
      e_out[row * pe + l16 + 16 * eo] = ecur;
    }
#pragma unroll
    for (int e = eo + 1; e < EPL; ++e)
#pragma unroll
      for (int lo = 0; lo < 16; ++lo)
        x[e] = fma(-eb[lo], static_cast<double>(rl[eo * 16 + lo][l16 * EPL + e]), x[e]);
  }
}

// Tile of W[rows, cols] -= E R[k0 .. k0 + K, cols] on float64 MFMA
// (v_mfma_f64_16x16x4f64): TM x TN output tile at (i0, j0), 4 waves in a
// WR x WC grid, each a grid of 16 x 16 blocks. The accumulators start as the
// W tile (read at entry, under the first chunk's loads) and -E goes into LDS,
// so the MFMAs produce W - E R directly and the exit only stores. k advances
// in chunks of 16 through two LDS buffers held k-major ([k][row], [k][column]);
// the next chunk is loaded into registers (R converted to float64 on its way
// into LDS) while the current one is multiplied. E rows have pitch pe; columns
// run to col_end (a multiple of 32); rows past dout read as zero and are not
// written.
constexpr int kTK = 16;  // k chunk

// Row pitch TM + 16 (TN + 16) doubles: the four k rows one MFMA operand read
// touches fall on disjoint bank halves.
template <int TM, int TN>
struct TileLds {
  double as[2][kTK][TM + 16];
  double bs[2][kTK][TN + 16];
};

template <int K, int TM, int TN, int WR, int WC>
__device__ __forceinline__ void tile_role(TileLds<TM, TN>& sm, double* __restrict__ w, const float* __restrict__ r,
                                          const double* __restrict__ e, int64_t pe, int64_t dout, int64_t din,
                                          int64_t col_end, int64_t k0, int64_t i0, int64_t j0) {
  static_assert(WR * WC == 4 && TM % (16 * WR) == 0 && TN % (16 * WC) == 0, "tile shape");
  constexpr int BM = TM / WR / 16, BN = TN / WC / 16;  // 16 x 16 blocks per wave
  constexpr int DA = TM / 16;                          // doubles of E per thread per chunk
  static_assert(DA % 2 == 0 && (kTK * TN) % 256 == 0, "chunk shape");
  const int mv = static_cast<int>(dout - i0 < TM ? dout - i0 : TM);
  const int nv = static_cast<int>(col_end - j0 < TN ? col_end - j0 : TN);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = wave / WC, wj = wave % WC;
  // this thread's loads: E row ar, k offset ak (DA doubles); R elements tid + 256 q of the
  // kTK x TN chunk (row (tid + 256 q) / TN, column (tid + 256 q) % TN): consecutive lanes,
  // consecutive columns, in global memory and in LDS
  const int ar = tid / (kTK / DA), ak = (tid % (kTK / DA)) * DA;
  constexpr int NR = kTK * TN / 256;
  const int bc = tid % TN, bk0 = tid / TN;
  constexpr int BKS = 256 / TN;  // R rows between a thread's elements
  const bool a_ok = ar < mv, b_ok = bc < nv;
  const double* ap = e + (i0 + (a_ok ? ar : 0)) * pe + ak;
  const float* bp = r + (k0 + bk0) * din + j0 + (b_ok ? bc : 0);
  // two register sets: the chunk two ahead loads while one is multiplied and one waits
  double2 va[2][DA / 2];
  float vb[2][NR];
  // The loads are unconditional (ap and bp are clamped into the tile) and the out-of-range
  // operands are zeroed when stored to LDS: a load under a per-lane condition compiles to a
  // branch, and the wait for a prefetched chunk then also waits for every later load.
  auto load = [&](int set, int kc) {
#pragma unroll
    for (int q = 0; q < DA / 2; ++q) va[set][q] = *reinterpret_cast<const double2*>(ap + kc + 2 * q);
#pragma unroll
    for (int q = 0; q < NR; ++q) vb[set][q] = bp[int64_t(kc + q * BKS) * din];
  };
  auto store = [&](int set, int buf) {
#pragma unroll
    for (int q = 0; q < DA / 2; ++q) {
      sm.as[buf][ak + 2 * q][ar] = a_ok ? -va[set][q].x : 0.0;
      sm.as[buf][ak + 2 * q + 1][ar] = a_ok ? -va[set][q].y : 0.0;
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) sm.bs[buf][bk0 + q * BKS][bc] = b_ok ? vb[set][q] : 0.0f;
  };
  // D[i][j] of a 16 x 16 float64 block: lane l, register q -> i = 4 q + l / 16, j = l % 16
  // (measured on gfx950; the operands are A[i][k] at lane i + 16 k and B[k][j] at lane j + 16 k)
  const int jl = lane & 15, il = lane >> 4;
  f64x4 acc[BM][BN];
#pragma unroll
  for (int x = 0; x < BM; ++x)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = wi * (TM / WR) + x * 16 + 4 * q + il;
      const double* wr = w + (i0 + (i < mv ? i : 0)) * din + j0;
#pragma unroll
      for (int y = 0; y < BN; ++y) {
        const int j = wj * (TN / WC) + y * 16 + jl;
        acc[x][y][q] = wr[j < nv ? j : 0];
      }
    }
  constexpr int nchunk = K / kTK;
  load(0, 0);
  if (nchunk > 1) load(1, kTK);
  store(0, 0);
  __syncthreads();
#pragma unroll
  for (int ch = 0; ch < nchunk; ++ch) {
    const int buf = ch & 1;
    if (ch + 2 < nchunk) load(ch & 1, (ch + 2) * kTK);  // set ch & 1 was stored to LDS before this chunk
#pragma unroll
    for (int kk = 0; kk < kTK / 4; ++kk) {
      const int kr = 4 * kk + il;
      double fa[BM], fb[BN];
#pragma unroll
      for (int x = 0; x < BM; ++x) fa[x] = sm.as[buf][kr][wi * (TM / WR) + x * 16 + jl];
#pragma unroll
      for (int y = 0; y < BN; ++y) fb[y] = sm.bs[buf][kr][wj * (TN / WC) + y * 16 + jl];
#pragma unroll
      for (int x = 0; x < BM; ++x)
#pragma unroll
        for (int y = 0; y < BN; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    if (ch + 1 < nchunk) store((ch + 1) & 1, buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < BM; ++x)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = wi * (TM / WR) + x * 16 + 4 * q + il;
#pragma unroll
      for (int y = 0; y < BN; ++y) {
        const int j = wj * (TN / WC) + y * 16 + jl;
        if (i < mv && j < nv) w[(i0 + i) * din + j0 + j] = acc[x][y][q];
      }
    }
}

// One step of the sweep, two-level: blocks of B columns are grouped in
// super-blocks of sb blocks (sb = kSB where the float64 W'' is larger than the
// Infinity Cache; sb = 1, every launch updating every later column, where it
// fits: there the far updates hit the cache and the three launches of a
// super-block with little far work would leave the sweep's latency exposed). Workgroups [0, n_sweep) apply the errors no earlier
// launch applied to block [c0, c0 + B) and sweep it (errors to e_out); the others
// apply earlier errors to columns beyond the block, in 128 x 128 tiles:
//   * inside a super-block: the previous block's errors (rank B) to the rest of
//     the super-block, [c0 + B, super-block end);
//   * at a super-block's first block: the whole previous super-block's errors
//     (rank sb B) to every column from c0 + B on.
// So the columns right of a super-block are read and written once per super-block
// instead of once per block; each block still receives every earlier error before
// its sweep (the previous super-block's in its own launch at a super-block start,
// the earlier blocks of its own super-block through the far updates of the
// launches between). The roles touch disjoint columns, so the latency-bound sweep
// shares the GPU with the MFMA-bound update.
constexpr int kFT = 128;  // far tile edge
constexpr int kSB = 4;    // blocks per super-block

template <int B>
union StepLds {
  SweepLds<B> sw;
  TileLds<kFT, kFT> tl;
};

// Two waves per SIMD: a sweep workgroup and a far-update workgroup share each CU.
// TL: two-level (super-blocks); the one-level kernel carries only the rank-B far tile.
template <int B, bool SG, bool TL>
__global__ __launch_bounds__(256, 2) void obs_step_kernel(double* __restrict__ w, const float* __restrict__ r,
                                                   int64_t dout, int64_t din, int64_t c0, int bits, int group,
                                                   uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                   uint8_t* __restrict__ zeros, double* __restrict__ preround,
                                                   const double* __restrict__ e_near, int nq,
                                                   double* __restrict__ e_out, int pe, const double* __restrict__ e_far,
                                                   int kfar, int64_t far_end, int n_sweep, int far_cols) {
  __shared__ StepLds<B> sm;
  const int b = blockIdx.x;
  if (b < n_sweep) {
    sweep_role<B, SG, TL>(sm.sw, b, w, r, dout, din, c0, bits, group, codes, scales, zeros, preround, e_near, nq,
                          e_out, pe);
    return;
  }
  const int t = b - n_sweep;
  const int64_t i0 = int64_t(t / far_cols) * kFT, j0 = c0 + B + int64_t(t % far_cols) * kFT;
  if constexpr (TL) {
    if (kfar == kSB) {
      tile_role<kSB * B, kFT, kFT, 2, 2>(sm.tl, w, r, e_far, pe, dout, din, far_end, c0 - kSB * B, i0, j0);
      return;
    }
  }
  tile_role<B, kFT, kFT, 2, 2>(sm.tl, w, r, e_far, pe, dout, din, far_end, c0 - B, i0, j0);
}

// Super-block size: kSB where the float64 W'' (dout x din) exceeds the 256 MB Infinity Cache.
inline int super_blocks(int64_t dout, int64_t din) { return dout * din * 8 > (int64_t(256) << 20) ? kSB : 1; }

template <int B>
kq_status run_blocks(double* w, const float* r, int64_t dout, int64_t din, int bits, int group, uint8_t* codes,
                     float* scales, uint8_t* zeros, double* preround, double* e, hipStream_t st) {
  const int n_sweep = static_cast<int>((dout + kRowsPerWg - 1) / kRowsPerWg);
  const int far_rows = static_cast<int>((dout + kFT - 1) / kFT);
  // errors of two consecutive super-blocks, rows of nsb B
  const int nsb = super_blocks(dout, din);
  const int pe = nsb * B;
  double* ebuf[2] = {e, e + dout * pe};
  kq_status s;
  for (int64_t c0 = 0, k = 0; c0 < din; c0 += B, ++k) {
    const int64_t sb = k / nsb, j = k % nsb;
    double* e_cur = ebuf[sb & 1];
    const double* e_near = nullptr;
    const double* e_far = nullptr;
    int nq = 0, kfar = 1;
    int64_t far_end = c0 + B;
    if (k > 0 && j == 0) {  // super-block start: the whole previous super-block
      e_near = ebuf[(sb + 1) & 1];
      nq = nsb;
      e_far = e_near;
      kfar = nsb;
      far_end = din;
    } else if (j > 0) {      // inside a super-block: the previous block, to the rest of the super-block
      e_near = e_cur + (j - 1) * B;
      nq = 1;
      e_far = e_near;
      kfar = 1;
      far_end = (sb + 1) * nsb * B < din ? (sb + 1) * nsb * B : din;
    }
    const int far_cols = far_end > c0 + B ? static_cast<int>((far_end - c0 - B + kFT - 1) / kFT) : 0;
    {
      LaunchTimer timer("obs_step_kernel", st);
      const bool small_group = group > 0 && group < 16;  // groups that start inside a 16-column slice
      auto kern = nsb > 1 ? (small_group ? obs_step_kernel<B, true, true> : obs_step_kernel<B, false, true>)
                          : (small_group ? obs_step_kernel<B, true, false> : obs_step_kernel<B, false, false>);
      hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(n_sweep + far_cols * far_rows)), dim3(256), 0, st, w, r,
                         dout, din, c0, bits, group, codes, scales, zeros, preround, e_near, nq, e_cur + j * B, pe,
                         e_far, kfar, far_end, n_sweep, far_cols);
    }
    if ((s = check_launch("obs_step_kernel")) != KQ_OK) return s;
  }
  return KQ_OK;
}

}  // namespace

size_t obs_workspace(int64_t dout, int64_t din, int block) {
  (void)din;
  return align_up(2 * size_t(dout) * kSB * block * sizeof(double), 256);  // errors of two consecutive super-blocks
}

kq_status obs_run(double* w, const float* r, int64_t dout, int64_t din, int bits, int group, int block,
                  uint8_t* codes, float* scales, uint8_t* zeros, double* preround, void* ws, hipStream_t st) {
  double* e = static_cast<double*>(ws);
  if (group == 0) {
    {
      LaunchTimer timer("row_grid_kernel", st);
      hipLaunchKernelGGL(row_grid_kernel, dim3(static_cast<unsigned>((dout + 3) / 4)), dim3(256), 0, st, w, dout, din,
                         bits, scales, zeros);
    }
    kq_status s = check_launch("row_grid_kernel");
    if (s != KQ_OK) return s;
  }
  switch (block) {
    case 32: return run_blocks<32>(w, r, dout, din, bits, group, codes, scales, zeros, preround, e, st);
    case 64: return run_blocks<64>(w, r, dout, din, bits, group, codes, scales, zeros, preround, e, st);
    case 128: return run_blocks<128>(w, r, dout, din, bits, group, codes, scales, zeros, preround, e, st);
    default: return fail(KQ_EUNSUPPORTED, "block %d", block);
  }
}

}  // namespace kq
