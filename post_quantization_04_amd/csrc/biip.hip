// Bidirectional incoherence processing: diagonal rescale and randomised
// Hadamard rotation of W on both sides, with H_X and H_G transformed alongside.
//
// The rotation of an n = m * 2^k vector is U = (Q_m kron H_p / sqrt(p)) diag(sigma):
// a sign flip, a length-p fast Walsh-Hadamard transform on each of the m
// contiguous chunks and an m x m mix across chunks at equal offsets. The two
// factors act on different index parts, so their order does not matter; the
// inverse applies Q_m^T and puts the sign flip last.
//
// A two-sided transform U_L M U_R^T needs every element of M on both sides:
//   * column direction: "digit" passes, one thread per column and 256
//     consecutive columns per workgroup; a pass holds the 2^6 rows that differ
//     in six bits of the row index in registers and applies that part of the
//     Walsh-Hadamard transform, a last pass applies the odd-factor mix across
//     the rows at stride p. The Hadamard factors and the mix act on different
//     index bits, so they commute. Per-row and per-column factors cost one
//     uniform and one per-thread load here, so these passes carry the
//     diagonal scales of both sides;
//   * row direction (contiguous): one workgroup per row; radix-16 butterflies
//     in registers over windows of four index bits, the row staged in LDS
//     between windows (two exchanges for a 4096-long row), the odd mix on the
//     staged row. This pass carries only the signs of its side.
// Forward: column passes first (signs and scales at their first load), then
// the row pass (signs at load, 1 / sqrt(p) at store). Inverse: row pass first
// (signs at store), then the column passes (signs and scales at the last store).
// Butterflies and mixes run in float64 registers; values between passes are
// float32 (the precision of H and of the rotated weight the sweep needs); the
// final W'' is written in float64.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kRowThreads = 512;   // rot_rows (general row kernel)
constexpr int kFwThreads = 256;    // row_fwht, rows whose staging leaves room for several workgroups per CU
constexpr int kFwThreadsWide = 1024;  // row_fwht, rows staged in more than half of the LDS (one workgroup per CU)
constexpr int kColThreads = 256;
constexpr size_t kRowLdsF64 = 64 * 1024;  // row_fwht keeps float64 in LDS up to this size
constexpr size_t kLdsBudget = 160 * 1024;  // bytes of LDS a pass may use (all of a gfx950 CU)
// Register array sizes for the odd-factor mix: instantiations for m = 1 (no
// mix), m <= 7 and m <= 63 keep the common no-mix case light.

struct Rot {
  const int8_t* signs;  // nullptr: no rotation on this axis
  const double* q;
  int m;
  int log2p;
  int inverse;          // apply U^T instead of U
  double out_scale;     // 1 / sqrt(p)
};

struct Scales {
  const double* row;    // per-row factor (nullable)
  const double* col;    // per-column factor (nullable)
  int at_store;         // apply when storing instead of when loading
};

template <typename T>
__device__ __forceinline__ double load_elem(const T* p);
template <>
__device__ __forceinline__ double load_elem<uint16_t>(const uint16_t* p) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(*p) << 16));
}
template <>
__device__ __forceinline__ double load_elem<float>(const float* p) {
  return static_cast<double>(*p);
}
template <>
__device__ __forceinline__ double load_elem<double>(const double* p) {
  return *p;
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, double v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, double v) {
  *p = static_cast<float>(v);
}
template <>
__device__ __forceinline__ void store_elem<double>(double* p, double v) {
  *p = v;
}

// Buffer-resource access: a uniform base (SGPRs) plus a 32-bit per-lane and a
// 32-bit uniform byte offset, so that a thread's many row accesses share one
// address register. Reads at or past num_records return 0 and writes there are
// dropped.
using Rsrc = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(n),
                                           0x00020000);
}

template <typename T>
__device__ __forceinline__ double bload(Rsrc r, uint32_t voff, uint32_t soff);
template <>
__device__ __forceinline__ double bload<uint16_t>(Rsrc r, uint32_t voff, uint32_t soff) {
  return static_cast<double>(
      __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)) << 16));
}
template <>
__device__ __forceinline__ double bload<float>(Rsrc r, uint32_t voff, uint32_t soff) {
  return static_cast<double>(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0)));
}
template <>
__device__ __forceinline__ double bload<double>(Rsrc r, uint32_t voff, uint32_t soff) {
  const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return __hiloint2double(static_cast<int>(u[1]), static_cast<int>(u[0]));
}

template <typename T>
__device__ __forceinline__ T bload_raw(Rsrc r, uint32_t voff, uint32_t soff);
template <>
__device__ __forceinline__ uint16_t bload_raw<uint16_t>(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
template <>
__device__ __forceinline__ float bload_raw<float>(Rsrc r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
template <>
__device__ __forceinline__ double bload_raw<double>(Rsrc r, uint32_t voff, uint32_t soff) {
  return bload<double>(r, voff, soff);
}
__device__ __forceinline__ double widen(uint16_t x) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(x) << 16));
}
__device__ __forceinline__ double widen(float x) { return static_cast<double>(x); }
__device__ __forceinline__ double widen(double x) { return x; }

template <typename T>
__device__ __forceinline__ void bstore(Rsrc r, uint32_t voff, uint32_t soff, double v);
template <>
__device__ __forceinline__ void bstore<float>(Rsrc r, uint32_t voff, uint32_t soff, double v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(static_cast<float>(v)), r, voff, soff, 0);
}
template <>
__device__ __forceinline__ void bstore<double>(Rsrc r, uint32_t voff, uint32_t soff, double v) {
  using u2 = unsigned int __attribute__((__vector_size__(2 * sizeof(unsigned int))));
  u2 u;
  u[0] = static_cast<unsigned>(__double2loint(v));
  u[1] = static_cast<unsigned>(__double2hiint(v));
  __builtin_amdgcn_raw_buffer_store_b64(u, r, voff, soff, 0);
}

__device__ __forceinline__ double scale_factor(const Scales& sc, int64_t i, int64_t j) {
  double f = 1.0;
  if (sc.row) f *= sc.row[i];
  if (sc.col) f *= sc.col[j];
  return f;
}

// Length-p Walsh-Hadamard butterflies on every chunk; element t of vector c at buf[t * C + c].
template <typename T>
__device__ void fwht_lds(T* buf, int n, int log2c, int log2p) {
  const int C = 1 << log2c;
  const int half = (n << log2c) >> 1;
  for (int s = 0; s < log2p; ++s) {
    const int h = 1 << s;
    for (int idx = threadIdx.x; idx < half; idx += blockDim.x) {
      const int c = idx & (C - 1);
      const int pr = idx >> log2c;
      const int i = ((pr >> s) << (s + 1)) + (pr & (h - 1));
      const T x = buf[(i << log2c) + c];
      const T y = buf[((i + h) << log2c) + c];
      buf[(i << log2c) + c] = x + y;
      buf[((i + h) << log2c) + c] = x - y;
    }
    __syncthreads();
  }
}

// y[a] = sum_k Q[a][k] v[k] (or Q[k][a]) across the m chunks, at each offset b and vector c.
// A thread holds one (b, c) column of m values in registers and writes the m
// outputs back in place; Q is read from global memory at wave-uniform
// addresses (scalar loads). The register array has the bucket size MB >= m.
template <typename T, int MB>
__device__ __forceinline__ void mix_column(T* base, int stride, int m, const double* __restrict__ q,
                                           int transpose) {
  T v[MB];
#pragma unroll
  for (int k = 0; k < MB; ++k) v[k] = (k < m) ? base[k * stride] : T(0);
  const int qs_a = transpose ? 1 : m, qs_k = transpose ? m : 1;
  for (int a = 0; a < m; ++a) {
    const double* qa = q + a * qs_a;
    double acc = 0.0;
    // k >= m: v[k] is zero and the Q index is clamped inside the row, so the term adds zero
#pragma unroll
    for (int k = 0; k < MB; ++k) acc = fma(qa[(k < m ? k : m - 1) * qs_k], static_cast<double>(v[k]), acc);
    base[a * stride] = static_cast<T>(acc);
  }
}

template <typename T, int MB>
__device__ void mix_lds(T* buf, int log2c, int m, int log2p, const double* q, int transpose) {
  const int C = 1 << log2c;
  const int p = 1 << log2p;
  const int total = p << log2c;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int c = idx & (C - 1);
    const int b = idx >> log2c;
    mix_column<T, MB>(buf + (b << log2c) + c, p << log2c, m, q, transpose);
  }
  __syncthreads();
}

template <typename T, int MB>
__device__ void transform_lds(T* buf, int n, int log2c, const Rot& rot) {
  if (!rot.signs) return;
  fwht_lds(buf, n, log2c, rot.log2p);
  if (MB > 1 && rot.m > 1) mix_lds<T, MB>(buf, log2c, rot.m, rot.log2p, rot.q, rot.inverse);
}

// One row per workgroup; the transform runs along the row (length n).
template <typename T, typename Src, typename Dst, int MB>
__global__ __launch_bounds__(kRowThreads) void rot_rows(const Src* __restrict__ src, int64_t lds, int64_t n,
                                                        Dst* __restrict__ dst, int64_t ldd, Rot rot, Scales sc) {
  extern __shared__ double smem[];
  T* buf = reinterpret_cast<T*>(smem);
  const int64_t row = blockIdx.x;
  const Src* s = src + row * lds;
  for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
    double v = load_elem<Src>(s + j);
    if (!sc.at_store) v *= scale_factor(sc, row, j);
    if (rot.signs && !rot.inverse) v *= static_cast<double>(rot.signs[j]);
    buf[j] = static_cast<T>(v);
  }
  __syncthreads();
  transform_lds<T, MB>(buf, static_cast<int>(n), 0, rot);
  Dst* o = dst + row * ldd;
  const double os = rot.signs ? rot.out_scale : 1.0;
  for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
    double v = static_cast<double>(buf[j]) * os;
    if (rot.signs && rot.inverse) v *= static_cast<double>(rot.signs[j]);
    if (sc.at_store) v *= scale_factor(sc, row, j);
    store_elem<Dst>(o + j, v);
  }
}

// Row direction for rows of n = m * 2^k values with k >= 8 (every chunk holds
// whole groups of 16). Window w covers index bits [lo, lo + 4) of the offset
// inside a chunk; a thread takes a group of the 16 offsets that differ only in
// those bits and applies the four radix-2 stages in registers. Window 0 reads
// 16 contiguous values straight from global memory, the last window writes
// straight to global memory (consecutive threads, consecutive offsets); the
// row is staged in LDS in between, with one pad slot per 16 values so that
// strided groups spread over the banks. When k is not a multiple of 4 the
// last window is moved down to [k - 4, k) and skips the stages already done.
struct RowFw {
  int k;                 // log2 p
  int m;                 // odd factor
  const double* q;       // m x m, row-major (m > 1)
  int transpose;         // apply Q^T
  const int8_t* signs;   // [n], along the row
  int inverse;           // signs (and factors) at store instead of at load
  double out_scale;      // 1 / sqrt(p)
  const double* rowf;    // per-row factor (nullable), same side as the signs
  const double* colf;    // per-column factor (nullable), same side as the signs
};

__device__ __forceinline__ int lpad(int e) { return e + (e >> 4); }

// Stands in for an absent per-column factor: indexed with stride 0, so that the factor's load
// never sits under a condition (a conditional load compiles to a branch whose result is waited
// for at once, which serializes the loads of a group).
__device__ double kUnitFactor = 1.0;

template <typename Src>
__device__ __forceinline__ void load16(const Src* p, double v[16]);
template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, double v[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  const uint4 a = q[0], b = q[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = static_cast<double>(__uint_as_float(w[i] << 16));
    v[2 * i + 1] = static_cast<double>(__uint_as_float(w[i] & 0xffff0000u));
  }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, double v[16]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = q[i];
    v[4 * i] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
}
template <>
__device__ __forceinline__ void load16<double>(const double* p, double v[16]) {
  const double2* q = reinterpret_cast<const double2*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double2 f = q[i];
    v[2 * i] = f.x;
    v[2 * i + 1] = f.y;
  }
}

// Bit i set: sign i of the 16 at p is negative (each sign byte is +1 or -1).
__device__ __forceinline__ uint32_t neg_mask16(const int8_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m |= ((w[i >> 2] >> (8 * (i & 3) + 7)) & 1u) << i;
  return m;
}

// x with its sign flipped when bit b of m is set.
__device__ __forceinline__ double flip(double x, uint32_t m, int b) {
  const int hi = __double2hiint(x) ^ static_cast<int>(((m >> b) & 1u) << 31);
  return __hiloint2double(hi, __double2loint(x));
}

// Radix-2 stages j = first .. 3 on a group of 16 (element t differs from t + 2^j in bit j).
__device__ __forceinline__ void bfly16(double v[16], int first) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j >= first) {
      const int h = 1 << j;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        if (t & h) continue;
        const double a = v[t], b = v[t + h];
        v[t] = a + b;
        v[t + h] = a - b;
      }
    }
  }
}

// Window 0 of group e0 (16 contiguous values v, as loaded): signs and factors when they go at
// load, the first four radix-2 stages, then the values into the row's LDS slots.
template <typename T>
__device__ __forceinline__ void row_stage0(T* buf, int e0, double v[16], const RowFw& rf, double rowf,
                                           const double* colf, int cstep) {
  if (!rf.inverse) {
    const uint32_t neg = neg_mask16(rf.signs + e0);
    // the factors of the 16 values are contiguous (16-byte loads from one base) or all one
    // (cstep = 0, a uniform branch): 16 separate addresses would take 32 registers
    double cf[16];
    if (cstep) {
      const double2* c2 = reinterpret_cast<const double2*>(colf + e0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double2 t = c2[i];
        cf[2 * i] = t.x;
        cf[2 * i + 1] = t.y;
      }
    } else {
      const double c = colf[0];
#pragma unroll
      for (int i = 0; i < 16; ++i) cf[i] = c;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = flip(v[i] * (rowf * cf[i]), neg, i);
  }
  bfly16(v, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[lpad(e0 + i)] = static_cast<T>(v[i]);
}

// The rest of a row once window 0 is in LDS: the odd mix on the staged row, the windows above
// bit 4 through LDS, and the last window's values to global memory at o.
template <typename T, typename Dst, int MB, int NT>
__device__ __forceinline__ void row_rest(T* buf, Dst* o, int64_t n, const RowFw& rf, double rowf,
                                         const double* colf, int cstep) {
  const int k = rf.k, kg = k - 4;
  const int ng = static_cast<int>(n >> 4);
  __syncthreads();
  if (MB > 1 && rf.m > 1) {
    const int p = 1 << k;
    for (int b = threadIdx.x; b < p; b += NT)
      mix_column<T, MB>(buf + lpad(b), p + (p >> 4), rf.m, rf.q, rf.transpose);
    __syncthreads();
  }
  const Rsrc ro = make_rsrc(o, uint64_t(n) * sizeof(Dst));
  for (int lo = 4; lo < k; lo += 4) {
    const bool last = lo + 4 >= k;
    const int wlo = last ? k - 4 : lo;   // >= 4: a group's LDS slots are a0 + i * lstep
    const int first = lo - wlo;
    const int lstep = (1 << wlo) + (1 << (wlo - 4));
    const uint32_t gstep = uint32_t(sizeof(Dst)) << wlo;
    for (int g = threadIdx.x; g < ng; g += NT) {
      const int a = g >> kg, idx = g & ((1 << kg) - 1);
      const int e0 = (a << k) + (idx & ((1 << wlo) - 1)) + ((idx >> wlo) << (wlo + 4));
      T* b0 = buf + lpad(e0);
      double v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = static_cast<double>(b0[i * lstep]);
      bfly16(v, first);
      if (!last) {
#pragma unroll
        for (int i = 0; i < 16; ++i) b0[i * lstep] = static_cast<T>(v[i]);
      } else {
        const uint32_t vo = uint32_t(e0) * uint32_t(sizeof(Dst));
        if (rf.inverse) {
          double f[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int e = e0 + (i << wlo);
            f[i] = static_cast<double>(rf.signs[e]) * (rowf * colf[e * cstep]);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) bstore<Dst>(ro, vo, i * gstep, v[i] * rf.out_scale * f[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) bstore<Dst>(ro, vo, i * gstep, v[i] * rf.out_scale);
        }
      }
    }
    if (!last) __syncthreads();
  }
}

template <typename T, typename Src, typename Dst, int MB, int NT>
__global__ __launch_bounds__(NT, NT == kFwThreads ? 6 : 1) void row_fwht(const Src* __restrict__ src, int64_t lds, int64_t n,
                                                       Dst* __restrict__ dst, int64_t ldd, RowFw rf) {
  extern __shared__ double smem[];
  T* buf = reinterpret_cast<T*>(smem);
  const int64_t row = blockIdx.x;
  const int ng = static_cast<int>(n >> 4);
  const Src* s = src + row * lds;
  const double rowf = rf.rowf ? rf.rowf[row] : 1.0;
  const double* colf = rf.colf ? rf.colf : &kUnitFactor;
  const int cstep = rf.colf ? 1 : 0;
  for (int g = threadIdx.x; g < ng; g += NT) {
    double v[16];
    load16<Src>(s + (g << 4), v);
    row_stage0<T>(buf, g << 4, v, rf, rowf, colf, cstep);
  }
  row_rest<T, Dst, MB, NT>(buf, dst + row * ldd, n, rf, rowf, colf, cstep);
}

// One digit pass of the column direction on a [n_rows, n_cols] row-major
// matrix, in LDS (used for odd factors above 31). Workgroup g x column tile
// ct transforms the tile of rows r(a, i) = base(g) + a * sa + i * si
// (a < mt, i < 2^lp) and columns
// [ct * TC, ct * TC + TC): Walsh-Hadamard butterflies over i, then the odd
// mix over a. Elementwise steps (sign, scales, 1 / sqrt(p)) are applied at
// load or at store as the pass's position in the transform requires.
struct ColPass {
  int64_t n_rows, n_cols;
  int64_t lds, ldd;            // row pitch (elements) of the source and of the destination
  int lo, hishift;             // base row of group g: (g mod 2^lo) + (g / 2^lo) * 2^hishift
  int64_t si, sa;
  int lp, mt;
  const double* q;             // mt x mt, row-major (mt > 1)
  int transpose;               // apply Q^T
  // elementwise factors (passes with OPS): value *= rl[r] * cl[j] at load and rs[r] * cs[j] at store
  const double* rl;
  const double* cl;
  const double* rs;
  const double* cs;
};

__device__ __forceinline__ int64_t group_base(const ColPass& cp, int64_t g) {
  return (g & ((int64_t(1) << cp.lo) - 1)) + ((g >> cp.lo) << cp.hishift);
}

template <int TC>
__device__ __forceinline__ int64_t tile_row(const ColPass& cp, int64_t base, int li) {
  const int a = li >> cp.lp, i = li & ((1 << cp.lp) - 1);
  return base + a * cp.sa + i * cp.si;
}

template <typename Src, typename Dst, int MB, int TC>
__global__ __launch_bounds__(kColThreads) void col_pass(const Src* __restrict__ src, Dst* __restrict__ dst,
                                                        ColPass cp) {
  extern __shared__ double smem[];
  constexpr int P = TC + 1;  // LDS row pitch (doubles)
  double* tile = smem;
  const int pt = 1 << cp.lp;
  const int L = cp.mt << cp.lp;
  const int nct = static_cast<int>((cp.n_cols + TC - 1) / TC);
  const int64_t g = blockIdx.x / nct;
  const int64_t c0 = int64_t(blockIdx.x % nct) * TC;
  const int64_t base = group_base(cp, g);
  const int tid = threadIdx.x;
  for (int e = tid; e < L * TC; e += kColThreads) {
    const int c = e % TC, li = e / TC;
    const int64_t r = tile_row<TC>(cp, base, li);
    const int64_t j = c0 + c;
    double v = 0.0;
    if (j < cp.n_cols) v = load_elem<Src>(src + r * cp.lds + j) * (cp.rl[r] * cp.cl[j]);
    tile[li * P + c] = v;
  }
  __syncthreads();
  // butterflies over i for every (a, column)
  const int half = (L * TC) >> 1;
  for (int s = 0; s < cp.lp; ++s) {
    const int h = 1 << s;
    for (int idx = tid; idx < half; idx += kColThreads) {
      const int c = idx % TC, pr = idx / TC;
      const int a = pr >> (cp.lp - 1), ip = pr & ((pt >> 1) - 1);
      const int i = ((ip >> s) << (s + 1)) + (ip & (h - 1));
      double* x0 = tile + (a * pt + i) * P + c;
      double* x1 = x0 + h * P;
      const double u = *x0, w = *x1;
      *x0 = u + w;
      *x1 = u - w;
    }
    __syncthreads();
  }
  if (MB > 1 && cp.mt > 1) {
    for (int idx = tid; idx < pt * TC; idx += kColThreads) {
      const int c = idx % TC, i = idx / TC;
      mix_column<double, MB>(tile + i * P + c, pt * P, cp.mt, cp.q, cp.transpose);
    }
    __syncthreads();
  }
  for (int e = tid; e < L * TC; e += kColThreads) {
    const int c = e % TC, li = e / TC;
    const int64_t r = tile_row<TC>(cp, base, li);
    const int64_t j = c0 + c;
    if (j >= cp.n_cols) continue;
    store_elem<Dst>(dst + r * cp.ldd + j, tile[li * P + c] * (cp.rs[r] * cp.cs[j]));
  }
}

// Elementwise factors of a column transform: rows (r < n_rows) and columns
// (j < n_cols) at load and at store. Load side: sigma_r (forward) and the
// load-side scales; store side: 1 / sqrt(p), sigma_r (inverse) and the
// store-side scales. Unused factors are ones.
__global__ void factors_kernel(int64_t n_rows, int64_t n_cols, const int8_t* __restrict__ signs, int inverse,
                               double out_scale, Scales sc, double* __restrict__ rl, double* __restrict__ cl,
                               double* __restrict__ rs, double* __restrict__ cs) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n_rows) {
    const double sg = signs ? static_cast<double>(signs[i]) : 1.0;
    const double row = sc.row ? sc.row[i] : 1.0;
    rl[i] = (signs && !inverse ? sg : 1.0) * (sc.at_store ? 1.0 : row);
    rs[i] = out_scale * (signs && inverse ? sg : 1.0) * (sc.at_store ? row : 1.0);
  }
  if (i < n_cols) {
    const double col = sc.col ? sc.col[i] : 1.0;
    cl[i] = sc.at_store ? 1.0 : col;
    cs[i] = sc.at_store ? col : 1.0;
  }
}

// Column-direction passes in registers: one thread per column, 256
// consecutive columns per workgroup (each wave reads 512 contiguous bytes
// per row), the L rows of the thread's group held in registers; no LDS and
// no barriers. col_fwht applies 2^LP-point butterflies over rows
// base(g) + i * si; col_mix applies the odd mix over rows base(g) + a * sa.

// Value of x in lane l of the wave.
__device__ __forceinline__ double lane_value(double x, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), l);
  return __hiloint2double(hi, lo);
}

// Launches cover column blocks [cb0, cb0 + ncb) of every group. PARTIAL: the
// one block that runs past the last column; its extra lanes leave at once.
template <typename Src, typename Dst, int LP, bool OPS, bool PARTIAL>
__global__ __launch_bounds__(kColThreads) void col_fwht(const Src* __restrict__ src, Dst* __restrict__ dst,
                                                        ColPass cp, int64_t cb0, int64_t ncb) {
  constexpr int L = 1 << LP;
  const int64_t g = blockIdx.x / ncb;
  const int64_t j0 = (cb0 + blockIdx.x % ncb) * kColThreads;  // uniform
  const uint32_t lane = threadIdx.x;
  if (PARTIAL && j0 + lane >= cp.n_cols) return;
  const int64_t base = group_base(cp, g);
  // rows base + t * si of this block: buffer bases at row base, byte offsets t * step + lane * element size
  const Rsrc rs_src = make_rsrc(src + base * cp.lds + j0, uint64_t((L - 1) * cp.si * cp.lds + kColThreads) * sizeof(Src));
  const Rsrc rs_dst = make_rsrc(dst + base * cp.ldd + j0, uint64_t((L - 1) * cp.si * cp.ldd + kColThreads) * sizeof(Dst));
  const uint32_t sstep = static_cast<uint32_t>(cp.si * cp.lds * int64_t(sizeof(Src)));
  const uint32_t dstep = static_cast<uint32_t>(cp.si * cp.ldd * int64_t(sizeof(Dst)));
  const uint32_t lo_s = lane * uint32_t(sizeof(Src)), lo_d = lane * uint32_t(sizeof(Dst));
  // per-row factors: in full blocks lane t of each wave holds row t's, broadcast with readlane
  const int wl = static_cast<int>(lane & 63);
  double rl = 1.0, rs = 1.0, cl = 1.0, cs = 1.0;
  if (OPS) {
    if (!PARTIAL && wl < L) {
      rl = cp.rl[base + wl * cp.si];
      rs = cp.rs[base + wl * cp.si];
    }
    cl = cp.cl[j0 + lane];
    cs = cp.cs[j0 + lane];
  }
  // loads land as raw values (one register each for 16/32-bit types); each half of the
  // rows is then widened and transformed on its own before the last stage joins them
  Src raw[L];
#pragma unroll
  for (int t = 0; t < L; ++t) raw[t] = bload_raw<Src>(rs_src, lo_s, t * sstep);
  double v[L];
  constexpr int H = L > 1 ? L / 2 : 1;
#pragma unroll
  for (int half = 0; half < (L > 1 ? 2 : 1); ++half) {
#pragma unroll
    for (int t = half * H; t < half * H + H; ++t) {
      v[t] = widen(raw[t]);
      if (OPS) v[t] *= (PARTIAL ? cp.rl[base + t * cp.si] : lane_value(rl, t)) * cl;
    }
#pragma unroll
    for (int st = 0; st + 1 < LP; ++st) {
      const int h = 1 << st;
#pragma unroll
      for (int t = half * H; t < half * H + H; ++t) {
        if (t & h) continue;
        const double a = v[t], b = v[t + h];
        v[t] = a + b;
        v[t + h] = a - b;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (LP > 0) {
#pragma unroll
    for (int t = 0; t < H; ++t) {
      const double a = v[t], b = v[t + H];
      v[t] = a + b;
      v[t + H] = a - b;
    }
  }
#pragma unroll
  for (int t = 0; t < L; ++t) {
    const double f = OPS ? (PARTIAL ? cp.rs[base + t * cp.si] : lane_value(rs, t)) * cs : 1.0;
    bstore<Dst>(rs_dst, lo_d, t * dstep, OPS ? v[t] * f : v[t]);
  }
}

// Column blocks of 256 a col_mix thread covers: four for mixes of up to 7 (28 loads in flight
// per thread; one block each left the pass waiting on load latency), one for wider mixes.
template <int MB>
constexpr int mix_cols() { return MB <= 8 ? 4 : 1; }

template <typename Src, typename Dst, int MB, bool OPS>
__global__ __launch_bounds__(kColThreads) void col_mix(const Src* __restrict__ src, Dst* __restrict__ dst,
                                                       ColPass cp) {
  constexpr int CPT = mix_cols<MB>();
  const int64_t span = int64_t(kColThreads) * CPT;
  const int64_t ncb = (cp.n_cols + span - 1) / span;
  const int64_t g = blockIdx.x / ncb;
  const int64_t j0 = (blockIdx.x % ncb) * span + threadIdx.x;  // column of block 0
  const int64_t base = group_base(cp, g);
  const int m = cp.mt;
  // every slot loads (slots past m read row m - 1 again and are zeroed after; columns past the
  // end read the last column and are not stored), so all loads are in flight together: a load
  // under a condition compiles to a branch that waits for it
  int64_t jc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) jc[c] = j0 + c * kColThreads < cp.n_cols ? j0 + c * kColThreads : cp.n_cols - 1;
  Src raw[CPT][MB];
  double rf[MB], cl[CPT], cs[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    cl[c] = OPS ? cp.cl[jc[c]] : 1.0;
    cs[c] = OPS ? cp.cs[jc[c]] : 1.0;
  }
#pragma unroll
  for (int a = 0; a < MB; ++a) {
    const int64_t r = base + (a < m ? a : m - 1) * cp.sa;
#pragma unroll
    for (int c = 0; c < CPT; ++c) raw[c][a] = src[r * cp.lds + jc[c]];
    rf[a] = OPS ? cp.rl[r] : 1.0;
  }
  const int qs_a = cp.transpose ? 1 : m, qs_k = cp.transpose ? m : 1;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t j = j0 + c * kColThreads;
    double v[MB];
#pragma unroll
    for (int a = 0; a < MB; ++a) v[a] = a < m ? widen(raw[c][a]) * (OPS ? rf[a] * cl[c] : 1.0) : 0.0;
    if (j >= cp.n_cols) continue;
#pragma unroll
    for (int a = 0; a < MB; ++a) {
      if (a < m) {
        const double* qa = cp.q + a * qs_a;
        double acc = 0.0;
        // k >= m: v[k] is zero and the Q index is clamped inside the row, so the term adds zero
#pragma unroll
        for (int k = 0; k < MB; ++k) acc = fma(qa[(k < m ? k : m - 1) * qs_k], v[k], acc);
        const int64_t r = base + a * cp.sa;
        store_elem<Dst>(dst + r * cp.ldd + j, OPS ? acc * (cp.rs[r] * cs[c]) : acc);
      }
    }
  }
}

// s_i = H_ii^(1/4) (1 where H_ii <= 0 or the side is off) and its reciprocal.
__global__ void scales_kernel(const float* __restrict__ h, int64_t n, int enabled, double* __restrict__ s,
                              double* __restrict__ inv) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  double v = 1.0;
  if (enabled) {
    const double d = static_cast<double>(h[i * n + i]);
    if (d > 0.0) v = sqrt(sqrt(d));
  }
  s[i] = v;
  inv[i] = 1.0 / v;
}

__global__ void recip_kernel(const double* __restrict__ s, int64_t n, double* __restrict__ inv) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) inv[i] = 1.0 / s[i];
}

Rot make_rot(const kq_rot* r, bool on, bool inverse) {
  Rot o{};
  if (!on) return o;
  o.signs = r->signs;
  o.q = r->q;
  o.m = r->m;
  o.log2p = r->log2p;
  o.inverse = inverse ? 1 : 0;
  o.out_scale = 1.0 / sqrt(static_cast<double>(int64_t(1) << r->log2p));
  return o;
}

// Bytes of LDS for a row of n elements of type T.
template <typename T>
size_t lds_bytes(int64_t n, const Rot&) { return size_t(n) * sizeof(T); }

template <typename T>
bool fits(int64_t n, const Rot& rot) { return lds_bytes<T>(n, rot) <= kLdsBudget; }

template <typename K>
kq_status allow_lds(K kernel, const char* name) {
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(kLdsBudget)) != hipSuccess)
    return fail(KQ_EDEVICE, "%s: cannot raise the LDS limit to %zu bytes", name, kLdsBudget);
  return KQ_OK;
}

// Mix bucket of an odd factor: 1 (none), 8 (m <= 7), 32 (m <= 31) or 64 (m <= 63).
inline int mix_bucket(int m) { return m == 1 ? 1 : (m <= 7 ? 8 : (m <= 31 ? 32 : 64)); }

template <typename T, typename Src, typename Dst, int MB>
kq_status launch_rows_mb(const Src* src, int64_t lds, int64_t rows, int64_t n, Dst* dst, int64_t ldd, Rot rot,
                         Scales sc, hipStream_t st) {
  auto kern = rot_rows<T, Src, Dst, MB>;
  kq_status r = allow_lds(kern, "rot_rows");
  if (r != KQ_OK) return r;
  {
    LaunchTimer timer("rot_rows", st);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(rows)), dim3(kRowThreads), lds_bytes<T>(n, rot), st, src, lds,
                       n, dst, ldd, rot, sc);
  }
  return check_launch("rot_rows");
}

template <typename T, typename Src, typename Dst>
kq_status launch_rows_t(const Src* src, int64_t lds, int64_t rows, int64_t n, Dst* dst, int64_t ldd, Rot rot,
                        Scales sc, hipStream_t st) {
  switch (mix_bucket(rot.signs ? rot.m : 1)) {
    case 1: return launch_rows_mb<T, Src, Dst, 1>(src, lds, rows, n, dst, ldd, rot, sc, st);
    case 8: return launch_rows_mb<T, Src, Dst, 8>(src, lds, rows, n, dst, ldd, rot, sc, st);
    case 32: return launch_rows_mb<T, Src, Dst, 32>(src, lds, rows, n, dst, ldd, rot, sc, st);
    default: return launch_rows_mb<T, Src, Dst, 64>(src, lds, rows, n, dst, ldd, rot, sc, st);
  }
}

template <typename T, typename Src, typename Dst, int MB>
kq_status launch_fw_mb(const Src* src, int64_t lds, int64_t rows, int64_t n, Dst* dst, int64_t ldd, const RowFw& rf,
                       size_t lds_bytes, hipStream_t st) {
  // a row staged in more than half of the LDS leaves one workgroup per CU: it gets 16 waves, so that
  // the CU still has enough loads in flight (4 waves stalled on them at 28672-long rows)
  const bool wide = lds_bytes > kLdsBudget / 2;
  auto kern = wide ? row_fwht<T, Src, Dst, MB, kFwThreadsWide> : row_fwht<T, Src, Dst, MB, kFwThreads>;
  kq_status r = allow_lds(kern, "row_fwht");
  if (r != KQ_OK) return r;
  {
    LaunchTimer timer("row_fwht", st);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(rows)), dim3(wide ? kFwThreadsWide : kFwThreads), lds_bytes, st,
                       src, lds, n, dst, ldd, rf);
  }
  return check_launch("row_fwht");
}

template <typename T, typename Src, typename Dst>
kq_status launch_fw_t(const Src* src, int64_t lds, int64_t rows, int64_t n, Dst* dst, int64_t ldd, const RowFw& rf,
                      hipStream_t st) {
  const size_t bytes = size_t(n + (n >> 4)) * sizeof(T);
  switch (mix_bucket(rf.m)) {
    case 1: return launch_fw_mb<T, Src, Dst, 1>(src, lds, rows, n, dst, ldd, rf, bytes, st);
    case 8: return launch_fw_mb<T, Src, Dst, 8>(src, lds, rows, n, dst, ldd, rf, bytes, st);
    default: return launch_fw_mb<T, Src, Dst, 32>(src, lds, rows, n, dst, ldd, rf, bytes, st);
  }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Row direction of rot on each of the rows (pitches lds, ldd elements), with
// the diagonal factors of sc. The register-butterfly kernel takes chunks of at
// least 256, odd factors up to 31, 16-byte aligned rows, signs and column
// factors, and factors on the signs' side; anything else takes the LDS kernel.
template <typename Src, typename Dst>
kq_status launch_rows(const Src* src, int64_t lds, int64_t rows, int64_t n, Dst* dst, int64_t ldd, Rot rot,
                      Scales sc, hipStream_t st) {
  const bool side_ok = (!sc.row && !sc.col) || (sc.at_store != 0) == (rot.inverse != 0);
  const bool rows_aligned = aligned16(src) && (lds * int64_t(sizeof(Src))) % 16 == 0;
  if (rot.signs && rot.log2p >= 8 && rot.m <= 31 && side_ok && rows_aligned && aligned16(rot.signs) &&
      (!sc.col || aligned16(sc.col))) {
    const RowFw rf{rot.log2p, rot.m, rot.q, rot.inverse, rot.signs, rot.inverse, rot.out_scale, sc.row, sc.col};
    // float64 staging for float64 output while a row stays small; float32 staging (one
    // rounding per window, below the float32 output's own) keeps more rows per CU
    if (sizeof(Dst) == sizeof(double) && size_t(n + (n >> 4)) * sizeof(double) <= kRowLdsF64)
      return launch_fw_t<double>(src, lds, rows, n, dst, ldd, rf, st);
    if (size_t(n + (n >> 4)) * sizeof(float) <= kLdsBudget)
      return launch_fw_t<float>(src, lds, rows, n, dst, ldd, rf, st);
  }
  if (fits<double>(n, rot)) return launch_rows_t<double>(src, lds, rows, n, dst, ldd, rot, sc, st);
  return launch_rows_t<float>(src, lds, rows, n, dst, ldd, rot, sc, st);
}

template <typename Src, typename Dst, int MB, int TC>
kq_status launch_col_pass(const Src* src, Dst* dst, const ColPass& cp, int64_t groups, hipStream_t st) {
  auto kern = col_pass<Src, Dst, MB, TC>;
  kq_status r = allow_lds(kern, "col_pass");
  if (r != KQ_OK) return r;
  const int64_t L = int64_t(cp.mt) << cp.lp;
  const size_t lds = size_t(L * (TC + 1)) * sizeof(double);
  const int64_t nct = (cp.n_cols + TC - 1) / TC;
  {
    LaunchTimer timer("col_pass", st);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(groups * nct)), dim3(kColThreads), lds, st, src, dst, cp);
  }
  return check_launch("col_pass");
}

template <typename Src, typename Dst>
kq_status col_pass_any(const Src* src, Dst* dst, const ColPass& cp, int64_t groups, hipStream_t st) {
  const int64_t L = int64_t(cp.mt) << cp.lp;
  const bool wide = L <= 128;  // 64-column tiles while the tile stays small, else 32
  const int mb = mix_bucket(cp.mt);
  if (wide) {
    if (mb == 1) return launch_col_pass<Src, Dst, 1, 64>(src, dst, cp, groups, st);
    if (mb == 8) return launch_col_pass<Src, Dst, 8, 64>(src, dst, cp, groups, st);
    if (mb == 32) return launch_col_pass<Src, Dst, 32, 64>(src, dst, cp, groups, st);
    return launch_col_pass<Src, Dst, 64, 64>(src, dst, cp, groups, st);
  }
  if (mb == 1) return launch_col_pass<Src, Dst, 1, 32>(src, dst, cp, groups, st);
  if (mb == 8) return launch_col_pass<Src, Dst, 8, 32>(src, dst, cp, groups, st);
  if (mb == 32) return launch_col_pass<Src, Dst, 32, 32>(src, dst, cp, groups, st);
  return launch_col_pass<Src, Dst, 64, 32>(src, dst, cp, groups, st);
}

template <typename Src, typename Dst, int LP>
kq_status launch_fwht(const Src* src, Dst* dst, const ColPass& cp, bool ops, hipStream_t st) {
  const int64_t groups = cp.n_rows >> LP;
  const int64_t nfull = cp.n_cols / kColThreads;
  {
    LaunchTimer timer("col_fwht", st);
    if (nfull > 0) {
      const dim3 grid(static_cast<unsigned>(groups * nfull));
      if (ops) hipLaunchKernelGGL((col_fwht<Src, Dst, LP, true, false>), grid, dim3(kColThreads), 0, st, src, dst, cp,
                                  int64_t(0), nfull);
      else hipLaunchKernelGGL((col_fwht<Src, Dst, LP, false, false>), grid, dim3(kColThreads), 0, st, src, dst, cp,
                              int64_t(0), nfull);
    }
    if (cp.n_cols % kColThreads) {
      const dim3 grid(static_cast<unsigned>(groups));
      if (ops) hipLaunchKernelGGL((col_fwht<Src, Dst, LP, true, true>), grid, dim3(kColThreads), 0, st, src, dst, cp,
                                  nfull, int64_t(1));
      else hipLaunchKernelGGL((col_fwht<Src, Dst, LP, false, true>), grid, dim3(kColThreads), 0, st, src, dst, cp,
                              nfull, int64_t(1));
    }
  }
  return check_launch("col_fwht");
}

template <typename Src, typename Dst, int MB>
kq_status launch_mix(const Src* src, Dst* dst, const ColPass& cp, bool ops, hipStream_t st) {
  const int64_t span = int64_t(kColThreads) * mix_cols<MB>();
  const int64_t ncb = (cp.n_cols + span - 1) / span;
  const dim3 grid(static_cast<unsigned>((cp.n_rows / cp.mt) * ncb));
  {
    LaunchTimer timer("col_mix", st);
    if (ops) hipLaunchKernelGGL((col_mix<Src, Dst, MB, true>), grid, dim3(kColThreads), 0, st, src, dst, cp);
    else hipLaunchKernelGGL((col_mix<Src, Dst, MB, false>), grid, dim3(kColThreads), 0, st, src, dst, cp);
  }
  return check_launch("col_mix");
}

// One pass; ops: apply the pass's factor arrays (cp.rl .. cp.cs point at ones where unused).
template <typename Src, typename Dst>
kq_status col_step(const Src* src, Dst* dst, const ColPass& cp, bool ops, hipStream_t st) {
  if (cp.mt == 1) {
    switch (cp.lp) {
      case 0: return launch_fwht<Src, Dst, 0>(src, dst, cp, ops, st);
      case 1: return launch_fwht<Src, Dst, 1>(src, dst, cp, ops, st);
      case 2: return launch_fwht<Src, Dst, 2>(src, dst, cp, ops, st);
      case 3: return launch_fwht<Src, Dst, 3>(src, dst, cp, ops, st);
      case 4: return launch_fwht<Src, Dst, 4>(src, dst, cp, ops, st);
      case 5: return launch_fwht<Src, Dst, 5>(src, dst, cp, ops, st);
      default: return launch_fwht<Src, Dst, 6>(src, dst, cp, ops, st);
    }
  }
  if (cp.mt <= 7) return launch_mix<Src, Dst, 8>(src, dst, cp, ops, st);
  if (cp.mt <= 31) return launch_mix<Src, Dst, 32>(src, dst, cp, ops, st);
  return col_pass_any<Src, Dst>(src, dst, cp, cp.n_rows / cp.mt, st);  // m in 33 .. 63: LDS tile (always applies)
}

// Column direction of U_rot applied to a [n_rows, n_cols] matrix (n_rows = n of the rotation):
// butterfly passes over 6-bit chunks of the row index, then the odd mix, src -> mid -> ... -> dst
// with mid a float32 buffer (it may equal src when that is float32; every pass works in place
// on its own elements). Signs and load-side scales go with the first pass; the 1 / sqrt(p)
// factor, inverse signs and store-side scales with the last. fac holds 2 n_rows + 2 n_cols
// doubles for the factor arrays; ones has max(n_rows, n_cols) ones.
template <typename Src, typename Dst>
kq_status launch_cols(const Src* src, int64_t lds, int64_t n_rows, int64_t n_cols, Dst* dst, int64_t ldd, float* mid,
                      int64_t ldm, const Rot& rot, Scales sc, double* fac, const double* ones, hipStream_t st) {
  const int k = rot.signs ? rot.log2p : 0;
  const int m = rot.signs ? rot.m : 1;
  ColPass passes[4];
  int np = 0;
  for (int lo = 0; lo < k; lo += 6) {
    ColPass cp{};
    cp.lp = (k - lo < 6) ? k - lo : 6;
    cp.lo = lo;
    cp.hishift = lo + cp.lp;
    cp.si = int64_t(1) << lo;
    cp.mt = 1;
    passes[np++] = cp;
  }
  if (m > 1) {
    ColPass cp{};
    cp.lp = 0;
    cp.lo = k;  // groups enumerate the offset b inside a chunk
    cp.hishift = k;
    cp.si = 0;
    cp.sa = int64_t(1) << k;
    cp.mt = m;
    cp.q = rot.q;
    cp.transpose = rot.inverse;
    passes[np++] = cp;
  }
  if (np == 0) {  // no rotation on this axis: one elementwise pass
    ColPass cp{};
    cp.mt = 1;
    passes[np++] = cp;
  }
  double* rl = fac;
  double* rs = fac + n_rows;
  double* cl = fac + 2 * n_rows;
  double* cs = cl + n_cols;
  {
    const int64_t n = n_rows > n_cols ? n_rows : n_cols;
    LaunchTimer timer("factors_kernel", st);
    hipLaunchKernelGGL(factors_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, n_rows,
                       n_cols, rot.signs, rot.inverse, rot.signs ? rot.out_scale : 1.0, sc, rl, cl, rs, cs);
  }
  kq_status r = check_launch("factors_kernel");
  if (r != KQ_OK) return r;
  for (int i = 0; i < np; ++i) {
    passes[i].n_rows = n_rows;
    passes[i].n_cols = n_cols;
    passes[i].lds = i == 0 ? lds : ldm;
    passes[i].ldd = i == np - 1 ? ldd : ldm;
    passes[i].rl = i == 0 ? rl : ones;
    passes[i].cl = i == 0 ? cl : ones;
    passes[i].rs = i == np - 1 ? rs : ones;
    passes[i].cs = i == np - 1 ? cs : ones;
  }
  if (np == 1) return col_step<Src, Dst>(src, dst, passes[0], true, st);
  r = col_step<Src, float>(src, mid, passes[0], true, st);
  for (int i = 1; i + 1 < np && r == KQ_OK; ++i) r = col_step<float, float>(mid, mid, passes[i], false, st);
  if (r != KQ_OK) return r;
  return col_step<float, Dst>(mid, dst, passes[np - 1], true, st);
}

// Row pitch of the float32 intermediate for rows of n values: a multiple of 64
// values, moved off multiples of 1024 so that rows at power-of-two distances
// (the column passes step over 2^6 rows at a time) do not share memory channels.
int64_t mid_pitch(int64_t n) {
  const int64_t r = (n + 63) / 64 * 64;
  return r % 1024 == 0 ? r + 64 : r;
}

// U S^-1 M S^-1 U^T of a d x d float32 matrix, in place, through a float32 scratch copy:
// column passes (with both scales) h -> tmp, then the row pass tmp -> h. M need not be
// symmetric.
kq_status two_sided(float* h, int64_t d, const Rot& rot, const double* inv_s, float* tmp, double* fac,
                    const double* ones, hipStream_t st) {
  const int64_t pm = mid_pitch(d);
  kq_status r = launch_cols<float, float>(h, d, d, d, tmp, pm, tmp, pm, rot, Scales{inv_s, inv_s, 0}, fac, ones, st);
  if (r != KQ_OK) return r;
  return launch_rows<float, float>(tmp, pm, d, d, h, d, rot, Scales{nullptr, nullptr, 0}, st);
}

template <typename Src>
kq_status forward_w(const Src* w, int64_t dout, int64_t din, double* w_out, const Rot& ri, const Rot& ro,
                    const double* s_x, const double* s_g, float* tmp, double* fac, const double* ones,
                    hipStream_t st) {
  const Scales ld{s_g, s_x, 0};
  const Scales none{nullptr, nullptr, 0};
  const int64_t pm = mid_pitch(din);
  if (ri.signs && ro.signs) {
    kq_status r = launch_cols<Src, float>(w, din, dout, din, tmp, pm, tmp, pm, ro, ld, fac, ones, st);
    if (r != KQ_OK) return r;
    return launch_rows<float, double>(tmp, pm, dout, din, w_out, din, ri, none, st);
  }
  if (ro.signs) return launch_cols<Src, double>(w, din, dout, din, w_out, din, tmp, pm, ro, ld, fac, ones, st);
  return launch_rows<Src, double>(w, din, dout, din, w_out, din, ri, ld, st);  // ri may be "no rotation"
}

}  // namespace

// Workspace layout: float32 intermediate (the largest matrix), 1 / s_x, 1 / s_g, ...
static size_t biip_tmp_bytes(int64_t dout, int64_t din) {
  int64_t n = dout * mid_pitch(din);
  if (din * mid_pitch(din) > n) n = din * mid_pitch(din);
  if (dout * mid_pitch(dout) > n) n = dout * mid_pitch(dout);
  return align_up(size_t(n) * sizeof(float), 256);
}

// ... then the factor arrays of a column transform (4 max(dout, din)) and max(dout, din) ones.
static size_t biip_vec_bytes(int64_t n) { return align_up(size_t(n) * sizeof(double), 256); }

size_t biip_workspace(int64_t dout, int64_t din) {
  const int64_t nmax = dout > din ? dout : din;
  return biip_tmp_bytes(dout, din) + biip_vec_bytes(din) + biip_vec_bytes(dout) + biip_vec_bytes(4 * nmax) +
         biip_vec_bytes(nmax);
}

__global__ void ones_kernel(double* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 1.0;
}

kq_status biip_run(const void* w, int w_dtype, int64_t dout, int64_t din, double* w_out, float* h_x, float* h_g,
                   const kq_rot* rot_in, const kq_rot* rot_out, uint32_t flags, double* s_x, double* s_g,
                   void* ws, hipStream_t st) {
  const bool inp = flags & KQ_BIIP_INPUT, out = flags & KQ_BIIP_OUTPUT;
  const bool scale = flags & KQ_BIIP_SCALE, inverse = flags & KQ_BIIP_INVERSE;
  const int64_t nmax = dout > din ? dout : din;
  char* p = static_cast<char*>(ws);
  float* tmp = reinterpret_cast<float*>(p);
  p += biip_tmp_bytes(dout, din);
  double* inv_x = reinterpret_cast<double*>(p);
  p += biip_vec_bytes(din);
  double* inv_g = reinterpret_cast<double*>(p);
  p += biip_vec_bytes(dout);
  double* fac = reinterpret_cast<double*>(p);
  p += biip_vec_bytes(4 * nmax);
  double* ones = reinterpret_cast<double*>(p);
  kq_status r;
  {
    LaunchTimer timer("ones_kernel", st);
    hipLaunchKernelGGL(ones_kernel, dim3(static_cast<unsigned>((nmax + 255) / 256)), dim3(256), 0, st, ones, nmax);
  }
  if ((r = check_launch("ones_kernel")) != KQ_OK) return r;
  if (inverse) {
    {
      LaunchTimer timer("recip_kernel", st);
      hipLaunchKernelGGL(recip_kernel, dim3(static_cast<unsigned>((din + 255) / 256)), dim3(256), 0, st, s_x, din,
                         inv_x);
      hipLaunchKernelGGL(recip_kernel, dim3(static_cast<unsigned>((dout + 255) / 256)), dim3(256), 0, st, s_g, dout,
                         inv_g);
    }
    if ((r = check_launch("recip_kernel")) != KQ_OK) return r;
    // W = S_G^-1 U_G^T W'' U_X S_X^-1: input-side rows first, then output-side columns
    // with both scales at their last store (each scale follows the rotation of its index).
    const Rot ri = make_rot(rot_in, inp, true), ro = make_rot(rot_out, out, true);
    const double* w2 = static_cast<const double*>(w);
    const Scales at_store{inv_g, inv_x, 1};
    const int64_t pm = mid_pitch(din);
    if (out && inp) {
      r = launch_rows<double, float>(w2, din, dout, din, tmp, pm, ri, Scales{nullptr, nullptr, 1}, st);
      if (r != KQ_OK) return r;
      return launch_cols<float, double>(tmp, pm, dout, din, w_out, din, tmp, pm, ro, at_store, fac, ones, st);
    }
    if (out) return launch_cols<double, double>(w2, din, dout, din, w_out, din, tmp, pm, ro, at_store, fac, ones, st);
    return launch_rows<double, double>(w2, din, dout, din, w_out, din, ri, at_store, st);
  }
  // scales come from the raw diagonals, before H_X and H_G are transformed in place
  {
    LaunchTimer timer("scales_kernel", st);
    hipLaunchKernelGGL(scales_kernel, dim3(static_cast<unsigned>((din + 255) / 256)), dim3(256), 0, st, h_x, din,
                       (inp && scale) ? 1 : 0, s_x, inv_x);
  }
  if ((r = check_launch("scales_kernel")) != KQ_OK) return r;
  if (h_g || (out && scale)) {
    {
      LaunchTimer timer("scales_kernel", st);
      hipLaunchKernelGGL(scales_kernel, dim3(static_cast<unsigned>((dout + 255) / 256)), dim3(256), 0, st, h_g,
                         dout, (out && scale) ? 1 : 0, s_g, inv_g);
    }
  } else {
    {
      LaunchTimer timer("scales_kernel", st);
      hipLaunchKernelGGL(scales_kernel, dim3(static_cast<unsigned>((dout + 255) / 256)), dim3(256), 0, st,
                         static_cast<const float*>(nullptr), dout, 0, s_g, inv_g);
    }
  }
  if ((r = check_launch("scales_kernel")) != KQ_OK) return r;
  const Rot ri = make_rot(rot_in, inp, false), ro = make_rot(rot_out, out, false);
  switch (w_dtype) {
    case KQ_BF16:
      r = forward_w(static_cast<const uint16_t*>(w), dout, din, w_out, ri, ro, s_x, s_g, tmp, fac, ones, st);
      break;
    case KQ_F32:
      r = forward_w(static_cast<const float*>(w), dout, din, w_out, ri, ro, s_x, s_g, tmp, fac, ones, st);
      break;
    default:
      r = forward_w(static_cast<const double*>(w), dout, din, w_out, ri, ro, s_x, s_g, tmp, fac, ones, st);
      break;
  }
  if (r != KQ_OK) return r;
  if (inp && (r = two_sided(h_x, din, ri, inv_x, tmp, fac, ones, st)) != KQ_OK) return r;
  if (out && (r = two_sided(h_g, dout, ro, inv_g, tmp, fac, ones, st)) != KQ_OK) return r;
  return KQ_OK;
}

// M <- U S^-1 M S^-1 U^T for any square float32 M with given scales (the input-side map of
// H_X applied to another second-moment matrix of the same inputs), in place; workspace as
// for BiIP of an n x n weight.
kq_status biip_transform_run(float* m, int64_t n, const kq_rot* rot, const double* s, void* ws, hipStream_t st) {
  char* p = static_cast<char*>(ws);
  float* tmp = reinterpret_cast<float*>(p);
  p += biip_tmp_bytes(n, n);
  double* inv = reinterpret_cast<double*>(p);
  p += 2 * biip_vec_bytes(n);
  double* fac = reinterpret_cast<double*>(p);
  p += biip_vec_bytes(4 * n);
  double* ones = reinterpret_cast<double*>(p);
  kq_status r;
  {
    LaunchTimer timer("ones_kernel", st);
    hipLaunchKernelGGL(ones_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, ones, n);
    if (s)
      hipLaunchKernelGGL(recip_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, s, n, inv);
    else
      hipLaunchKernelGGL(ones_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, inv, n);
  }
  if ((r = check_launch("ones_kernel")) != KQ_OK) return r;
  return two_sided(m, n, make_rot(rot, true, false), inv, tmp, fac, ones, st);
}

}  // namespace kq
