// Bidirectional incoherence processing: diagonal rescale and randomised
// Hadamard rotation of W on both sides, with H_X and H_G transformed alongside.
//
// The rotation of an n = m * 2^k vector is U = (Q_m kron H_p / sqrt(p)) diag(sigma):
// a sign flip, a length-p fast Walsh-Hadamard transform on each of the m
// contiguous chunks and an m x m mix across chunks at equal offsets. The two
// factors act on different index parts, so their order does not matter; the
// inverse applies Q_m^T and puts the sign flip last.
//
// A two-sided transform U_L M U_R^T needs every element of M on both sides,
// so it takes two passes over HBM:
//   * row pass: one workgroup per row, the whole row in LDS (up to 32768
//     float32 values), transform along the row;
//   * column pass: one workgroup per panel of C adjacent columns, the whole
//     panel (n x C) in LDS, transform along the columns. Panels are handed
//     to XCDs in contiguous runs so that neighbouring panels, which share
//     cache lines, are read by the same L2.
// Butterflies and mixes run in float64 in LDS whenever the vector (or panel)
// fits (n <= 16384), else in float32; the intermediate between the passes is
// float64; scales are applied in float64 at load or store, and outputs are
// written in the destination precision.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kRowThreads = 512;
constexpr int kColThreads = 256;
constexpr size_t kLdsBudget = 160 * 1024;  // bytes of LDS a pass may use (all of a gfx950 CU)
constexpr int kMaxOdd = 64;                // register array size for the odd-factor mix

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
  int divide;           // use 1/s instead of s
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

__device__ __forceinline__ double scale_factor(const Scales& sc, int64_t i, int64_t j) {
  double f = 1.0;
  if (sc.row) f *= sc.row[i];
  if (sc.col) f *= sc.col[j];
  return sc.divide ? 1.0 / f : f;
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
template <typename T>
__device__ void mix_lds(T* buf, int log2c, int m, int log2p, const double* qs, int transpose) {
  const int C = 1 << log2c;
  const int p = 1 << log2p;
  const int total = p << log2c;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int c = idx & (C - 1);
    const int b = idx >> log2c;
    T v[kMaxOdd];
#pragma unroll
    for (int a = 0; a < kMaxOdd; ++a) v[a] = (a < m) ? buf[((a * p + b) << log2c) + c] : T(0);
    for (int a = 0; a < m; ++a) {
      T acc = T(0);
#pragma unroll
      for (int k = 0; k < kMaxOdd; ++k) {
        if (k < m) acc += static_cast<T>(transpose ? qs[k * m + a] : qs[a * m + k]) * v[k];
      }
      buf[((a * p + b) << log2c) + c] = acc;
    }
  }
  __syncthreads();
}

// float64 slots reserved for Q_m at the start of LDS.
__host__ __device__ inline int q_slots(const Rot& rot) { return rot.signs ? rot.m * rot.m : 0; }

__device__ void load_q(double* qs, const Rot& rot) {
  if (!rot.signs || rot.m == 1) return;
  for (int i = threadIdx.x; i < rot.m * rot.m; i += blockDim.x) qs[i] = rot.q[i];
}

template <typename T>
__device__ void transform_lds(T* buf, int n, int log2c, const Rot& rot, const double* qs) {
  if (!rot.signs) return;
  fwht_lds(buf, n, log2c, rot.log2p);
  if (rot.m > 1) mix_lds(buf, log2c, rot.m, rot.log2p, qs, rot.inverse);
}

// One row per workgroup; the transform runs along the row (length n).
template <typename T, typename Src, typename Dst>
__global__ __launch_bounds__(kRowThreads) void rot_rows(const Src* __restrict__ src, int64_t n,
                                                        Dst* __restrict__ dst, Rot rot, Scales sc) {
  extern __shared__ double smem[];
  double* qs = smem;
  T* buf = reinterpret_cast<T*>(smem + q_slots(rot));
  const int64_t row = blockIdx.x;
  load_q(qs, rot);
  const Src* s = src + row * n;
  for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
    double v = load_elem<Src>(s + j);
    if (!sc.at_store) v *= scale_factor(sc, row, j);
    if (rot.signs && !rot.inverse) v *= static_cast<double>(rot.signs[j]);
    buf[j] = static_cast<T>(v);
  }
  __syncthreads();
  transform_lds<T>(buf, static_cast<int>(n), 0, rot, qs);
  Dst* o = dst + row * n;
  const double os = rot.signs ? rot.out_scale : 1.0;
  for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
    double v = static_cast<double>(buf[j]) * os;
    if (rot.signs && rot.inverse) v *= static_cast<double>(rot.signs[j]);
    if (sc.at_store) v *= scale_factor(sc, row, j);
    store_elem<Dst>(o + j, v);
  }
}

// One panel of 2^log2c adjacent columns per workgroup; the transform runs
// along the columns (length n_rows). Matrix is [n_rows, n_cols] row-major.
template <typename T, typename Src, typename Dst>
__global__ __launch_bounds__(kColThreads) void rot_cols(const Src* __restrict__ src, int64_t n_rows,
                                                        int64_t n_cols, Dst* __restrict__ dst, int log2c,
                                                        int per_xcd, Rot rot, Scales sc) {
  extern __shared__ double smem[];
  double* qs = smem;
  T* buf = reinterpret_cast<T*>(smem + q_slots(rot));
  const int C = 1 << log2c;
  const int npanel = static_cast<int>((n_cols + C - 1) >> log2c);
  const int panel = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (panel >= npanel) return;
  const int64_t col0 = int64_t(panel) << log2c;
  load_q(qs, rot);
  const int64_t total = n_rows << log2c;
  for (int64_t idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int c = static_cast<int>(idx & (C - 1));
    const int64_t i = idx >> log2c;
    const int64_t j = col0 + c;
    double v = 0.0;
    if (j < n_cols) {
      v = load_elem<Src>(src + i * n_cols + j);
      if (!sc.at_store) v *= scale_factor(sc, i, j);
      if (rot.signs && !rot.inverse) v *= static_cast<double>(rot.signs[i]);
    }
    buf[idx] = static_cast<T>(v);
  }
  __syncthreads();
  transform_lds<T>(buf, static_cast<int>(n_rows), log2c, rot, qs);
  const double os = rot.signs ? rot.out_scale : 1.0;
  for (int64_t idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int c = static_cast<int>(idx & (C - 1));
    const int64_t i = idx >> log2c;
    const int64_t j = col0 + c;
    if (j >= n_cols) continue;
    double v = static_cast<double>(buf[idx]) * os;
    if (rot.signs && rot.inverse) v *= static_cast<double>(rot.signs[i]);
    if (sc.at_store) v *= scale_factor(sc, i, j);
    store_elem<Dst>(dst + i * n_cols + j, v);
  }
}

__global__ void scales_kernel(const float* __restrict__ h, int64_t n, int enabled, double* __restrict__ s) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  double v = 1.0;
  if (enabled) {
    const double d = static_cast<double>(h[i * n + i]);
    if (d > 0.0) v = sqrt(sqrt(d));
  }
  s[i] = v;
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

// Bytes of LDS for n elements of type T behind the Q_m slots.
template <typename T>
size_t lds_bytes(int64_t n, const Rot& rot) { return size_t(q_slots(rot)) * sizeof(double) + size_t(n) * sizeof(T); }

template <typename T>
bool fits(int64_t n, const Rot& rot) { return lds_bytes<T>(n, rot) <= kLdsBudget; }

// Widest power-of-two panel (<= 64 columns) whose n_rows x C block fits.
template <typename T>
int col_log2c(int64_t n_rows, const Rot& rot) {
  int l = 0;
  while (l < 6 && fits<T>(n_rows << (l + 1), rot)) ++l;
  return l;
}

template <typename T, typename K>
kq_status allow_lds(K kernel, const char* name) {
  static bool done = false;
  if (!done) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kLdsBudget)) != hipSuccess)
      return fail(KQ_EDEVICE, "%s: cannot raise the LDS limit to %zu bytes", name, kLdsBudget);
    done = true;
  }
  return KQ_OK;
}

template <typename Src, typename Dst>
kq_status launch_rows(const Src* src, int64_t rows, int64_t n, Dst* dst, Rot rot, Scales sc, hipStream_t st) {
  if (fits<double>(n, rot)) {
    kq_status r = allow_lds<double>(&rot_rows<double, Src, Dst>, "rot_rows");
    if (r != KQ_OK) return r;
    {
      LaunchTimer timer("rot_rows", st);
      hipLaunchKernelGGL((rot_rows<double, Src, Dst>), dim3(static_cast<unsigned>(rows)), dim3(kRowThreads),
                         lds_bytes<double>(n, rot), st, src, n, dst, rot, sc);
    }
  } else {
    kq_status r = allow_lds<float>(&rot_rows<float, Src, Dst>, "rot_rows");
    if (r != KQ_OK) return r;
    {
      LaunchTimer timer("rot_rows", st);
      hipLaunchKernelGGL((rot_rows<float, Src, Dst>), dim3(static_cast<unsigned>(rows)), dim3(kRowThreads),
                         lds_bytes<float>(n, rot), st, src, n, dst, rot, sc);
    }
  }
  return check_launch("rot_rows");
}

template <typename T, typename Src, typename Dst>
kq_status launch_cols_t(const Src* src, int64_t n_rows, int64_t n_cols, Dst* dst, Rot rot, Scales sc,
                        hipStream_t st) {
  const int log2c = col_log2c<T>(n_rows, rot);
  kq_status r = allow_lds<T>(&rot_cols<T, Src, Dst>, "rot_cols");
  if (r != KQ_OK) return r;
  const int npanel = static_cast<int>((n_cols + (1 << log2c) - 1) >> log2c);
  const int per_xcd = (npanel + kXcds - 1) / kXcds;
  {
    LaunchTimer timer("rot_cols", st);
    hipLaunchKernelGGL((rot_cols<T, Src, Dst>), dim3(static_cast<unsigned>(per_xcd * kXcds)), dim3(kColThreads),
                       lds_bytes<T>(n_rows << log2c, rot), st, src, n_rows, n_cols, dst, log2c, per_xcd, rot, sc);
  }
  return check_launch("rot_cols");
}

template <typename Src, typename Dst>
kq_status launch_cols(const Src* src, int64_t n_rows, int64_t n_cols, Dst* dst, Rot rot, Scales sc,
                      hipStream_t st) {
  if (fits<double>(n_rows, rot)) return launch_cols_t<double>(src, n_rows, n_cols, dst, rot, sc, st);
  return launch_cols_t<float>(src, n_rows, n_cols, dst, rot, sc, st);
}

// U M U^T of a symmetric d x d float32 matrix, in place, through a float64 scratch copy.
kq_status two_sided(float* h, int64_t d, const Rot& rot, const double* s, double* tmp, hipStream_t st) {
  Scales in{s, s, 1, 0};
  kq_status r = launch_rows<float, double>(h, d, d, tmp, rot, in, st);
  if (r != KQ_OK) return r;
  return launch_cols<double, float>(tmp, d, d, h, rot, Scales{nullptr, nullptr, 0, 0}, st);
}

template <typename Src>
kq_status forward_w(const Src* w, int64_t dout, int64_t din, double* w_out, const Rot& ri, const Rot& ro,
                    const double* s_x, const double* s_g, double* tmp, hipStream_t st) {
  const Scales ld{s_g, s_x, 0, 0};
  const Scales none{nullptr, nullptr, 0, 0};
  if (ri.signs && ro.signs) {
    kq_status r = launch_rows<Src, double>(w, dout, din, tmp, ri, ld, st);
    if (r != KQ_OK) return r;
    return launch_cols<double, double>(tmp, dout, din, w_out, ro, none, st);
  }
  if (ro.signs) return launch_cols<Src, double>(w, dout, din, w_out, ro, ld, st);
  return launch_rows<Src, double>(w, dout, din, w_out, ri, ld, st);  // ri may be "no rotation"
}

}  // namespace

size_t biip_workspace(int64_t dout, int64_t din) {
  int64_t n = dout * din;
  if (din * din > n) n = din * din;
  if (dout * dout > n) n = dout * dout;
  return align_up(size_t(n) * sizeof(double), 256);
}

kq_status biip_run(const void* w, int w_dtype, int64_t dout, int64_t din, double* w_out, float* h_x, float* h_g,
                   const kq_rot* rot_in, const kq_rot* rot_out, uint32_t flags, double* s_x, double* s_g,
                   void* ws, hipStream_t st) {
  const bool inp = flags & KQ_BIIP_INPUT, out = flags & KQ_BIIP_OUTPUT;
  const bool scale = flags & KQ_BIIP_SCALE, inverse = flags & KQ_BIIP_INVERSE;
  double* tmp = static_cast<double*>(ws);
  kq_status r;
  if (inverse) {
    // W = S_G^-1 U_G^T W'' U_X S_X^-1: input-side rows first, then output-side columns;
    // the row scale must follow the output-side rotation, which mixes rows.
    const Rot ri = make_rot(rot_in, inp, true), ro = make_rot(rot_out, out, true);
    const double* w2 = static_cast<const double*>(w);
    if (out) {
      r = launch_rows<double, double>(w2, dout, din, tmp, ri, Scales{nullptr, s_x, 1, 1}, st);
      if (r != KQ_OK) return r;
      return launch_cols<double, double>(tmp, dout, din, w_out, ro, Scales{s_g, nullptr, 1, 1}, st);
    }
    return launch_rows<double, double>(w2, dout, din, w_out, ri, Scales{s_g, s_x, 1, 1}, st);
  }
  // scales come from the raw diagonals, before H_X and H_G are transformed in place
  {
    LaunchTimer timer("scales_kernel", st);
    hipLaunchKernelGGL(scales_kernel, dim3(static_cast<unsigned>((din + 255) / 256)), dim3(256), 0, st, h_x, din,
                       (inp && scale) ? 1 : 0, s_x);
  }
  if ((r = check_launch("scales_kernel")) != KQ_OK) return r;
  if (h_g || (out && scale)) {
    {
      LaunchTimer timer("scales_kernel", st);
      hipLaunchKernelGGL(scales_kernel, dim3(static_cast<unsigned>((dout + 255) / 256)), dim3(256), 0, st, h_g,
                         dout, (out && scale) ? 1 : 0, s_g);
    }
  } else {
    {
      LaunchTimer timer("scales_kernel", st);
      hipLaunchKernelGGL(scales_kernel, dim3(static_cast<unsigned>((dout + 255) / 256)), dim3(256), 0, st,
                         static_cast<const float*>(nullptr), dout, 0, s_g);
    }
  }
  if ((r = check_launch("scales_kernel")) != KQ_OK) return r;
  const Rot ri = make_rot(rot_in, inp, false), ro = make_rot(rot_out, out, false);
  switch (w_dtype) {
    case KQ_BF16:
      r = forward_w(static_cast<const uint16_t*>(w), dout, din, w_out, ri, ro, s_x, s_g, tmp, st);
      break;
    case KQ_F32:
      r = forward_w(static_cast<const float*>(w), dout, din, w_out, ri, ro, s_x, s_g, tmp, st);
      break;
    default:
      r = forward_w(static_cast<const double*>(w), dout, din, w_out, ri, ro, s_x, s_g, tmp, st);
      break;
  }
  if (r != KQ_OK) return r;
  if (inp && (r = two_sided(h_x, din, ri, s_x, tmp, st)) != KQ_OK) return r;
  if (out && (r = two_sided(h_g, dout, ro, s_g, tmp, st)) != KQ_OK) return r;
  return KQ_OK;
}

}  // namespace kq
