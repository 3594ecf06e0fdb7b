// Packed codes and the decode matvec: y = S_G^-1 U_G^T W^'' U_X S_X^-1 x.
//
// The KronQ news item ("KronQ: Kronecker Hessians break GPTQ's 2-bit wall",
// deployment paragraph) describes the deployment path: the quantized weights
// ship as packed int4 / int2 codes and a single fused kernel dequantizes them
// and applies the BiIP rotations during the matvec; the KronQ article (Q&A,
// second question) puts the extra inference cost at two Hadamard transforms
// per layer, O(d log d) each.
//
// Packing: code j of a row sits in word j / (32 / c) at bits c (j mod 32 / c),
// with c = 2 for 2-bit codes, 4 for 3- and 4-bit codes, 8 above.
//
// Per call (one layer, or up to four layers that read the same input and share its input
// side: a block's q, k and v, or gate and up) and token batch (T <= 4 tokens), up to three
// launches on one stream:
//   1. input side, x1 = U_X S_X^-1 x (signs and scales on load, fast Walsh-Hadamard
//      transform per 2^k chunk in radix-16 register passes, odd-factor mix across the m
//      chunks on float32 MFMA): applied in LDS by every workgroup of the matvec while its
//      first rows are in flight when it has no odd factor and the grid is at most one
//      workgroup per CU, else as a one-workgroup (1024-thread) launch into the workspace;
//      skipped when there is neither a rotation nor a scale on that side;
//   2. the matvec over every layer's rows, 16 rows per 256-thread workgroup: every lane holds
//      the x1 entries of its words in registers, the four waves split each row's packed words (lane l of
//      wave w reads word 64 w + l + 256 i), dequantize on the fly,
//      y1[row] = sum_g s_g (sum_j q_j x1_j - z_g sum_j x1_j), one 32-bit load per word
//      and row, the loads of up to 16 rows in flight;
//   3. output sides, one 1024-thread workgroup per layer that has an output rotation:
//      transform per chunk, transposed odd mix, signs, 1 / s_g (a scale alone is applied by
//      the matvec).
// A side transform's data are small and its cost is round trips, not bytes: every global
// load of its first batch is issued before its first wait, and sides of whole groups of 16
// with aligned operands use 16-byte loads. (A fused last-workgroup output side needed a
// device-scope fence in every workgroup, which cost more than the launch.)
// Everything is float32; the float64 diagonal scales and rotation factors are rounded to
// float32 on load.
#include <mutex>

#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kThreads = 256;       // matvec workgroup
constexpr int kSideThreads = 1024;  // side-transform workgroup
constexpr int kRowsPerWg = 16;
constexpr int kQPitch = 64;         // LDS row pitch of a staged odd factor (e >> 6, e & 63 rely on it)
constexpr int kQFloats = 64 * kQPitch;  // staged odd factor: 64 rows (m <= 63, rows padded to 4)

typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ void pack_kernel(const uint8_t* __restrict__ codes, int64_t rows, int64_t cols, int c,
                            uint32_t* __restrict__ packed) {
  const int per = 32 / c;
  const int64_t wpr = cols / per;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * wpr) return;
  const int64_t r = idx / wpr, k = idx % wpr;
  const uint8_t* src = codes + r * cols + k * per;
  uint32_t w = 0;
  for (int t = 0; t < per; ++t) w |= uint32_t(src[t]) << (c * t);
  packed[idx] = w;
}

struct Side {
  int on;            // rotation applied
  int m, log2p;
  const int8_t* signs;
  const double* q;   // [m * m]
  const double* s;   // diagonal scale, NULL: 1
};

// One layer of a group that shares its input (q, k and v; gate and up).
struct Layer {
  const uint32_t* packed;
  const float* scales;
  const uint8_t* zeros;
  int64_t dout;
  float* y;           // [T, dout] final output (no output rotation) ...
  float* y1;          // ... or the matvec result before the output side
  const double* s_g;  // applied by the matvec when there is no output rotation
  int wg0;            // first matvec workgroup of this layer
};

struct DecodeArgs {
  Layer layer[KQ_DECODE_MAX_LAYERS];
  int n_layers;
  int64_t din;
  int group, ngroups;
  const float* x;     // [T, din]: x itself (fused input side) or x1 (separate or no input side)
  Side in;            // the input side, for the fused form
};

// Layer l of a kernel argument, read with constant indices only (a dynamic index into a
// by-value kernel argument makes the compiler copy it to scratch memory).
template <typename A, typename E>
__device__ __forceinline__ E pick(const A (&a)[KQ_DECODE_MAX_LAYERS], int l, E A::*f) {
  E v = a[0].*f;
#pragma unroll
  for (int k = 1; k < KQ_DECODE_MAX_LAYERS; ++k)
    if (l == k) v = a[k].*f;
  return v;
}

// Output sides of a group, one workgroup per layer that has one.
struct OutArgs {
  const float* src[KQ_DECODE_MAX_LAYERS];
  float* dst[KQ_DECODE_MAX_LAYERS];
  int n[KQ_DECODE_MAX_LAYERS];
  Side sd[KQ_DECODE_MAX_LAYERS];
};

// One pass of the fast Walsh-Hadamard transform over index bits [o, o + R) of every token's
// n entries (pitch n): a thread owns the 2^R entries of one group (indices that differ only in
// those bits) and does the R butterfly stages in registers.
template <int T, int R, int NT>
__device__ void fwht_pass(float* v, int n, int o) {
  constexpr int L = 1 << R;
  const int groups = n >> R, stride = 1 << o;
  for (int e = threadIdx.x; e < T * groups; e += NT) {
    const int t = e / groups, gidx = e - t * groups;
    const int base = ((gidx >> o) << (o + R)) | (gidx & (stride - 1));
    float* row = v + t * n + base;
    float a[L];
#pragma unroll
    for (int j = 0; j < L; ++j) a[j] = row[j * stride];
#pragma unroll
    for (int h = 1; h < L; h <<= 1)
#pragma unroll
      for (int j = 0; j < L; ++j)
        if ((j & h) == 0) {
          const float x = a[j], y = a[j + h];
          a[j] = x + y;
          a[j + h] = x - y;
        }
#pragma unroll
    for (int j = 0; j < L; ++j) row[j * stride] = a[j];
  }
  __syncthreads();
}

// H_p (unnormalised) on every chunk of p = 2^log2p entries of each token's n = m p entries,
// index bits [o0, log2p) (the bits below o0 already transformed).
template <int T, int NT>
__device__ void fwht_lds(float* v, int n, int log2p, int o0 = 0) {
  for (int o = o0; o < log2p; o += 4) {
    switch (log2p - o) {
      case 1: fwht_pass<T, 1, NT>(v, n, o); break;
      case 2: fwht_pass<T, 2, NT>(v, n, o); break;
      case 3: fwht_pass<T, 3, NT>(v, n, o); break;
      default: fwht_pass<T, 4, NT>(v, n, o); break;
    }
  }
}

// Odd-factor mix across the m chunks of p, in place: for every token t and column b of the
// m x p view of its vector, out[a] = sum_a' W[a][a'] v[a' p + b], with qs[a' * 64 + a] =
// W[a][a'] staged for all 64 x 64 entries (zero for a or a' >= m). A matrix product
// OUT = W V with V the m x (T p) matrix of the columns, on float32 MFMA (16 x 16 x 4): a wave
// takes one block of 16 columns and forms its four 16-row tiles (rows past m have zero weights,
// and only rows below m are stored); every wave reads its inputs before a barrier and writes
// after it, in rounds of whole column blocks.
template <int T, int NT, int KU>
__device__ void mix_mfma(float* v, int n, int m, int log2p, const float* qs) {
  constexpr int kWaves = NT / 64;
  constexpr int kMaxTiles = (KQ_MAX_ODD + 15) / 16;
  const int p = 1 << log2p;
  const int cols = T * p;
  const int mt = (m + 15) >> 4, kt = (m + 3) >> 2;
  const int nt = (cols + 15) >> 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lk = lane >> 4;
  for (int r0 = 0; r0 < nt; r0 += kWaves) {
    const int ni = r0 + wave;
    const int c = 16 * ni + li;                 // this lane's column (B operand and output)
    const bool cv = ni < nt && c < cols;
    float* col = v + (c >> log2p) * n + (c & (p - 1));
    floatx4 acc[kMaxTiles];
#pragma unroll
    for (int mi = 0; mi < kMaxTiles; ++mi) acc[mi] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (ni < nt) {
      // all kMaxTiles row tiles every step (rows past m have zero weights): no branch in the
      // loop, so the operand reads of the next steps are issued before the MFMAs wait on them
      // (KU K steps per iteration, written out: the staged weights are zero up to row 63)
      for (int k0 = 0; k0 < kt; k0 += KU) {
        float b[KU], a[KU][kMaxTiles];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          const int a2 = 4 * (k0 + u) + lk;     // input chunk of this lane's B entry
          b[u] = (cv && a2 < m) ? col[min(a2, m - 1) * p] : 0.0f;
#pragma unroll
          for (int mi = 0; mi < kMaxTiles; ++mi) a[u][mi] = qs[a2 * kQPitch + 16 * mi + li];  // W[16 mi + li][a2]
        }
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
          for (int mi = 0; mi < kMaxTiles; ++mi)
            acc[mi] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][mi], b[u], acc[mi], 0, 0, 0);
      }
    }
    __syncthreads();
    if (cv) {
      // lane holds column li, rows 4 lk + j of each 16-row tile
#pragma unroll
      for (int mi = 0; mi < kMaxTiles; ++mi) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int a = 16 * mi + 4 * lk + j;
          if (mi < mt && a < m) col[a * p] = acc[mi][j];
        }
      }
    }
    __syncthreads();
  }
}

// Stand-ins for an absent sign vector, scale vector or odd factor, so that the side kernel's
// loads never sit under a condition.
__device__ double kUnitScale = 1.0;
__device__ int8_t kPlusSign = 1;
__device__ __align__(16) double kUnitScales[16] = {1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0,
                                                   1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0};
__device__ __align__(16) int8_t kPlusSigns[16] = {1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1};

// One side of the rotation applied in LDS by the NT threads of a workgroup, for T tokens of n
// entries:
//   input side (OUT false):  (Q (x) H_p / sqrt p) diag(sigma) S^-1 src
//   output side (OUT true):  S^-1 diag(sigma) (Q^T (x) H_p / sqrt p) src
// (sd.on false: the scale alone). issue() requests the values, signs and scales of the first
// P * NT entries and the odd factor, all before the first wait; transform() stores them to LDS
// (the input side with sign and scale applied), streams any further entries, stages Q (times
// 1 / sqrt p) and runs the transform. On return lds[t n + i] times `tail` is the input side's
// result; the output side's entry i is lds[t n + i] * fo[k] for i = k NT + tid (first batch)
// and out_factor(i) beyond.
//
// Loads take clamped indices and are unconditional (entries past the end are never stored):
// a load under a per-lane condition becomes a branch whose result the compiler waits for
// before the next one, which would serialize the round trips.
template <int T, int NT, int P, bool OUT>
struct SideStage {
  static constexpr int kQPer = (kQFloats + NT - 1) / NT;
  const float* src;
  int n, nl, m;
  bool on, mixed;
  int log2p;
  const int8_t* sgp;
  int sgi;
  const double* svp;
  int svi;
  const double* qp;
  float post, tail;
  float val[P][T];
  int sg[P];
  double sv[P];
  double qv[kQPer];
  float fo[P];

  __device__ __forceinline__ void issue(const float* src_, int n_, const Side& sd) {
    const int tid = threadIdx.x;
    src = src_;
    n = n_;
    nl = n - 1;
    m = sd.m;
    on = sd.on != 0;
    mixed = on && m > 1;
    log2p = sd.log2p;
    sgp = on ? sd.signs : &kPlusSign;
    sgi = on ? 1 : 0;
    svp = sd.s ? sd.s : &kUnitScale;
    svi = sd.s ? 1 : 0;
    qp = sd.q ? sd.q : &kUnitScale;  // m = 1 without a rotation
    post = on ? 1.0f / sqrtf(static_cast<float>(1 << log2p)) : 1.0f;
    tail = (on && !mixed) ? post : 1.0f;  // 1 / sqrt(p) when not folded into Q
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int ic = min(k * NT + tid, nl);
#pragma unroll
      for (int t = 0; t < T; ++t) val[k][t] = src[t * n + ic];
    }
    const int ml = m - 1;
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int e = k * NT + tid;
      const int a2 = min(e >> 6, ml), a = min(e & (kQPitch - 1), ml);
      qv[k] = OUT ? qp[a2 * m + a] : qp[a * m + a2];
    }
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int ic = min(k * NT + tid, nl);
      sg[k] = sgp[ic * sgi];
      sv[k] = svp[ic * svi];
    }
  }

  __device__ __forceinline__ float out_factor(int i) const {
    const int ic = min(i, nl);
    return (sgp[ic * sgi] < 0 ? -tail : tail) / static_cast<float>(svp[ic * svi]);
  }

  __device__ __forceinline__ void transform(float* lds, float* qs) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int i = k * NT + tid;
      const float sgn = sg[k] < 0 ? -1.0f : 1.0f;
      fo[k] = OUT ? sgn * tail / static_cast<float>(sv[k]) : tail;
      if (i < n) {
        const float f = OUT ? 1.0f : sgn / static_cast<float>(sv[k]);
#pragma unroll
        for (int t = 0; t < T; ++t) lds[t * n + i] = val[k][t] * f;
      }
    }
    // entries past the first batch, one batch at a time
    for (int base = P * NT; base < n; base += P * NT) {
      float f[P];
#pragma unroll
      for (int k = 0; k < P; ++k) {
        const int ic = min(base + k * NT + tid, nl);
#pragma unroll
        for (int t = 0; t < T; ++t) val[k][t] = src[t * n + ic];
        const float sgn = sgp[ic * sgi] < 0 ? -1.0f : 1.0f;
        f[k] = OUT ? 1.0f : sgn / static_cast<float>(svp[ic * svi]);
      }
#pragma unroll
      for (int k = 0; k < P; ++k) {
        const int i = base + k * NT + tid;
        if (i < n) {
#pragma unroll
          for (int t = 0; t < T; ++t) lds[t * n + i] = val[k][t] * f[k];
        }
      }
    }
    if (mixed) {
      // all 64 rows (the product's K steps run in fours), zero outside the m x m factor
#pragma unroll
      for (int k = 0; k < kQPer; ++k) {
        const int e = k * NT + tid;
        const int a2 = e >> 6, a = e & (kQPitch - 1);
        if (e < kQFloats) qs[e] = (a < m && a2 < m) ? static_cast<float>(qv[k]) * post : 0.0f;
      }
    }
    __syncthreads();
    if (on) {
      fwht_lds<T, NT>(lds, n, log2p);
      if (mixed) mix_mfma<T, NT, (OUT && T >= 2) ? 2 : 4>(lds, n, m, log2p, qs);
    }
  }
};

// The same side with 16 consecutive entries per thread (a group), for n % 16 == 0 and 16-byte
// aligned values, signs and scales: a group's values, signs and scales arrive as 16-byte loads
// (a quarter of the instructions of one entry per load), and the first four butterfly stages
// (index bits 0..3, inside every chunk since 16 divides p) run in registers before the group
// goes to LDS, so the LDS passes start at bit 4. Group g = tid is requested by issue(); on
// return from transform() the output side's factors of that group are in fo[].
template <int T, int NT, bool OUT>
struct SideStageV {
  static constexpr int kQPer = (kQFloats + NT - 1) / NT;
  const float* src;
  int n, ng, m, log2p;
  bool on, mixed;
  const int8_t* sgp;
  int sgi;
  const double* svp;
  int svi;
  const double* qp;
  float post, tail;
  float val[T][16];
  uint4 sgw;
  double sv[16];
  double qv[kQPer];
  float fo[16];

  __device__ __forceinline__ void load_group(int g) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float4* p = reinterpret_cast<const float4*>(src + t * n + 16 * g);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 f = p[c];
        val[t][4 * c] = f.x;
        val[t][4 * c + 1] = f.y;
        val[t][4 * c + 2] = f.z;
        val[t][4 * c + 3] = f.w;
      }
    }
    sgw = *reinterpret_cast<const uint4*>(sgp + 16 * g * sgi);
    const double2* sp = reinterpret_cast<const double2*>(svp + 16 * g * svi);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const double2 d = sp[c];
      sv[2 * c] = d.x;
      sv[2 * c + 1] = d.y;
    }
  }

  __device__ __forceinline__ void issue(const float* src_, int n_, const Side& sd) {
    const int tid = threadIdx.x;
    src = src_;
    n = n_;
    ng = n >> 4;
    m = sd.m;
    on = sd.on != 0;
    mixed = on && m > 1;
    log2p = sd.log2p;
    sgp = on ? sd.signs : kPlusSigns;
    sgi = on ? 1 : 0;
    svp = sd.s ? sd.s : kUnitScales;
    svi = sd.s ? 1 : 0;
    qp = sd.q ? sd.q : &kUnitScale;
    post = on ? 1.0f / sqrtf(static_cast<float>(1 << log2p)) : 1.0f;
    tail = (on && !mixed) ? post : 1.0f;
    load_group(min(tid, ng - 1));
    const int ml = m - 1;
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int e = k * NT + tid;
      const int a2 = min(e >> 6, ml), a = min(e & (kQPitch - 1), ml);
      qv[k] = OUT ? qp[a2 * m + a] : qp[a * m + a2];
    }
  }

  // Signs and scales of the loaded group: applied to the values (input side) or kept as the
  // output factors (output side, first group only); then the group's four in-register
  // butterfly stages.
  template <bool KEEP>
  __device__ __forceinline__ void process_group() {
    const uint32_t w[4] = {sgw.x, sgw.y, sgw.z, sgw.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float sgn = ((w[j >> 2] >> (8 * (j & 3) + 7)) & 1u) ? -1.0f : 1.0f;
      if (OUT) {
        if (KEEP) fo[j] = sgn * tail / static_cast<float>(sv[j]);
      } else {
        const float f = sgn / static_cast<float>(sv[j]);
#pragma unroll
        for (int t = 0; t < T; ++t) val[t][j] *= f;
      }
    }
    if (on) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int h = 1; h < 16; h <<= 1)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if ((j & h) == 0) {
              const float x = val[t][j], y = val[t][j + h];
              val[t][j] = x + y;
              val[t][j + h] = x - y;
            }
    }
  }

  __device__ __forceinline__ void store_group(float* lds, int g) const {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float4* p = reinterpret_cast<float4*>(lds + t * n + 16 * g);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        p[c] = make_float4(val[t][4 * c], val[t][4 * c + 1], val[t][4 * c + 2], val[t][4 * c + 3]);
    }
  }

  __device__ __forceinline__ void transform(float* lds, float* qs) {
    const int tid = threadIdx.x;
    process_group<true>();
    if (tid < ng) store_group(lds, tid);
    // groups past the first NT, one at a time
    for (int g = tid + NT; g < ng; g += NT) {
      load_group(g);
      process_group<false>();
      store_group(lds, g);
    }
    if (mixed) {
#pragma unroll
      for (int k = 0; k < kQPer; ++k) {
        const int e = k * NT + tid;
        const int a2 = e >> 6, a = e & (kQPitch - 1);
        if (e < kQFloats) qs[e] = (a < m && a2 < m) ? static_cast<float>(qv[k]) * post : 0.0f;
      }
    }
    __syncthreads();
    if (on) {
      fwht_lds<T, NT>(lds, n, log2p, 4);
      if (mixed) mix_mfma<T, NT, (OUT && T >= 2) ? 2 : 4>(lds, n, m, log2p, qs);
    }
  }

  // Output factor of group g past the first NT (its signs and scales read again).
  __device__ __forceinline__ void out_factors(int g, float f[16]) const {
    const uint4 u = *reinterpret_cast<const uint4*>(sgp + 16 * g * sgi);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const double2* sp = reinterpret_cast<const double2*>(svp + 16 * g * svi);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const double2 d = sp[c];
      f[2 * c] = static_cast<float>(d.x);
      f[2 * c + 1] = static_cast<float>(d.y);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float sgn = ((w[j >> 2] >> (8 * (j & 3) + 7)) & 1u) ? -1.0f : 1.0f;
      f[j] = OUT ? sgn * tail / f[j] : tail;
    }
  }
};

// Floats of LDS a side transform of T x n entries uses: the entries, then Q at a 16-byte boundary.
__host__ __device__ constexpr int side_lds_floats(int n, int tokens) {
  return ((tokens * n + 3) & ~3) + kQFloats;
}

// One side for T tokens of n entries per 1024-thread workgroup: dst = S^-1 U^T src (output
// side, one workgroup per layer of a group) or U S^-1 src (input side, when it is not fused into
// the matvec; one workgroup). VEC: the grouped form (n % 16 == 0, every operand 16-byte aligned).
template <int T, bool OUT, bool VEC>
__global__ __launch_bounds__(kSideThreads) void side_kernel(OutArgs oa) {
  extern __shared__ float lds[];
  // workgroup l takes entry l (every member read with a constant index, then selected)
  const int l = blockIdx.x;
  const float* src = oa.src[0];
  float* dst = oa.dst[0];
  int n = oa.n[0];
  Side sd = oa.sd[0];
#pragma unroll
  for (int k = 1; k < KQ_DECODE_MAX_LAYERS; ++k)
    if (l == k) {
      src = oa.src[k];
      dst = oa.dst[k];
      n = oa.n[k];
      sd = oa.sd[k];
    }
  if constexpr (VEC) {
    SideStageV<T, kSideThreads, OUT> st;
    st.issue(src, n, sd);
    st.transform(lds, lds + side_lds_floats(n, T) - kQFloats);
    for (int g = threadIdx.x; g < st.ng; g += kSideThreads) {
      float f[16];
      if (g == static_cast<int>(threadIdx.x)) {
#pragma unroll
        for (int j = 0; j < 16; ++j) f[j] = OUT ? st.fo[j] : st.tail;
      } else {
        st.out_factors(g, f);
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float4* lp = reinterpret_cast<const float4*>(lds + t * n + 16 * g);
        float4* dp = reinterpret_cast<float4*>(dst + t * n + 16 * g);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 v = lp[c];
          dp[c] = make_float4(v.x * f[4 * c], v.y * f[4 * c + 1], v.z * f[4 * c + 2], v.w * f[4 * c + 3]);
        }
      }
    }
    return;
  }
  constexpr int P = 16 / T;
  SideStage<T, kSideThreads, P, OUT> st;
  st.issue(src, n, sd);
  st.transform(lds, lds + side_lds_floats(n, T) - kQFloats);
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const int i = k * kSideThreads + tid;
    if (i < n) {
#pragma unroll
      for (int t = 0; t < T; ++t) dst[t * n + i] = lds[t * n + i] * st.fo[k];
    }
  }
  for (int i = P * kSideThreads + tid; i < n; i += kSideThreads) {
    const float f = OUT ? st.out_factor(i) : st.tail;
#pragma unroll
    for (int t = 0; t < T; ++t) dst[t * n + i] = lds[t * n + i] * f;
  }
}

// Code k (k < 32 / C) of a packed word with C-bit containers, as a float.
template <int C>
__device__ __forceinline__ float code_at(uint32_t w, int k) {
  return static_cast<float>((w >> (C * k)) & ((1u << C) - 1u));
}

// Sum over the 64 lanes of a wave, returned uniform: DPP adds inside each row of 16 lanes
// (quad swaps, half-row and row mirrors), then the four row sums by readlane.
__device__ __forceinline__ float wave_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// C: container bits; CPL: codes per lane per row (din <= 256 CPL), held in registers with
// their x1 values; T: tokens (CPL T <= 64); IN: the input side is fused (applied in LDS by
// every workgroup), else x holds x1 already.
template <int C, int CPL, int T, bool IN>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs g) {
  extern __shared__ float lds[];  // the input side's vectors and odd factor, when it runs
  __shared__ float part[kRowsPerWg * 4 * T];
  constexpr int PER = 32 / C;          // codes per word
  constexpr int NW = CPL / PER;        // words per lane per row
  constexpr int U = NW <= 16 ? 16 / NW : 1;  // rows in flight: 16 words per lane
  static_assert(NW >= 1 && CPL % PER == 0 && PER % 4 == 0, "codes per lane");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this workgroup's layer: the last one whose first workgroup it has reached
  int li = 0;
#pragma unroll
  for (int l = 1; l < KQ_DECODE_MAX_LAYERS; ++l)
    if (l < g.n_layers && static_cast<int>(blockIdx.x) >= pick(g.layer, l, &Layer::wg0)) li = l;
  const uint32_t* packed = pick(g.layer, li, &Layer::packed);
  const float* scales = pick(g.layer, li, &Layer::scales);
  const uint8_t* zeros = pick(g.layer, li, &Layer::zeros);
  const int64_t dout = pick(g.layer, li, &Layer::dout);
  const int64_t din = g.din;
  const int64_t wpr = din / PER;  // words per row
  const int din32 = static_cast<int>(din);

  // Every load is unconditional, at a clamped index: a load under a per-lane condition becomes
  // a branch whose result the compiler waits for before the next one. Lanes past the end of a
  // row get x1 = 0 (so their words add nothing), and rows past dout are never stored.
  const int wl = static_cast<int>(wpr) - 1;
  int kw[NW], gcol[NW];
  bool kv[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int k = 64 * wave + lane + 256 * i;
    kv[i] = k <= wl;
    kw[i] = min(k, wl);
    gcol[i] = g.group ? (kw[i] * PER) / g.group : 0;
  }
  const int64_t r0 = int64_t(static_cast<int>(blockIdx.x) - pick(g.layer, li, &Layer::wg0)) * kRowsPerWg;
  uint32_t wd[U][NW], zr[U][NW];
  float sc[U][NW];
  auto load_rows = [&](int rb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = min(r0 + rb + u, dout - 1);
      const uint32_t* prow = packed + row * wpr;
      const float* srow = scales + row * g.ngroups;
      const uint8_t* zrow = zeros + row * g.ngroups;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        wd[u][i] = prow[kw[i]];
        sc[u][i] = srow[gcol[i]];
        zr[u][i] = zrow[gcol[i]];
      }
    }
  };

  // x1 = U_X S_X^-1 x for this lane's words k = 64 wave + lane + 256 i (PER consecutive entries
  // each). Fused input side: its loads first, then the first rows' (so that waiting for the
  // former leaves the latter in flight), then the transform in LDS, which every workgroup
  // repeats. Otherwise straight from x1, 16-byte aligned.
  float xv[NW][PER][T];
  if constexpr (IN) {
    SideStageV<T, kThreads, false> st;
    st.issue(g.x, din32, g.in);
    load_rows(0);
    st.transform(lds, lds + side_lds_floats(din32, T) - kQFloats);
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float4* src = reinterpret_cast<const float4*>(lds + t * din32 + kw[i] * PER);
#pragma unroll
        for (int c4 = 0; c4 < PER / 4; ++c4) {
          const float4 v = src[c4];
          xv[i][4 * c4][t] = v.x * st.tail;
          xv[i][4 * c4 + 1][t] = v.y * st.tail;
          xv[i][4 * c4 + 2][t] = v.z * st.tail;
          xv[i][4 * c4 + 3][t] = v.w * st.tail;
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float4* src = reinterpret_cast<const float4*>(g.x + t * din + int64_t(kw[i]) * PER);
#pragma unroll
        for (int c4 = 0; c4 < PER / 4; ++c4) {
          const float4 v = src[c4];
          xv[i][4 * c4][t] = v.x;
          xv[i][4 * c4 + 1][t] = v.y;
          xv[i][4 * c4 + 2][t] = v.z;
          xv[i][4 * c4 + 3][t] = v.w;
        }
      }
    load_rows(0);
  }
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int c = 0; c < PER; ++c)
#pragma unroll
      for (int t = 0; t < T; ++t) xv[i][c][t] = kv[i] ? xv[i][c][t] : 0.0f;
  float xs[NW][T];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float sum = 0.0f;
#pragma unroll
      for (int c = 0; c < PER; ++c) sum += xv[i][c][t];
      xs[i][t] = sum;
    }

  // rows r0 .. r0 + 15: partial sums per wave, U rows at a time
  for (int rb = 0; rb < kRowsPerWg; rb += U) {
    if (rb > 0) load_rows(rb);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[T];
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          float dot = 0.0f;
#pragma unroll
          for (int c = 0; c < PER; ++c) dot = fmaf(code_at<C>(wd[u][i], c), xv[i][c][t], dot);
          acc[t] = fmaf(sc[u][i], fmaf(-static_cast<float>(zr[u][i]), xs[i][t], dot), acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float v = wave_sum(acc[t]);
        if (lane == 0) part[((rb + u) * 4 + wave) * T + t] = v;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < kRowsPerWg * T; e += kThreads) {
    const int rr = e / T, t = e % T;
    const int64_t row = r0 + rr;
    if (row >= dout) continue;
    const float* pp = part + rr * 4 * T + t;
    const float v = (pp[0] + pp[T]) + (pp[2 * T] + pp[3 * T]);
    float* y1 = pick(g.layer, li, &Layer::y1);
    if (y1) {
      y1[t * dout + row] = v;
    } else {
      const double* s_g = pick(g.layer, li, &Layer::s_g);
      pick(g.layer, li, &Layer::y)[t * dout + row] = s_g ? v / static_cast<float>(s_g[row]) : v;
    }
  }
}

size_t side_lds_bytes(int64_t n, int64_t tokens) {
  return size_t(side_lds_floats(static_cast<int>(n), static_cast<int>(tokens))) * sizeof(float);
}

bool allow_lds(const void* fn, size_t bytes) {
  return bytes <= 64 * 1024 ||
         hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes)) == hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The grouped side form applies: whole groups of 16 and every operand 16-byte aligned.
bool side_vec_ok(const float* src, const float* dst, int64_t n, const Side& sd) {
  return n % 16 == 0 && aligned16(src) && (dst == nullptr || aligned16(dst)) && (!sd.on || aligned16(sd.signs)) &&
         (sd.s == nullptr || aligned16(sd.s));
}

// Side launch over `count` entries of oa (one workgroup each). The grouped form is used when
// every entry allows it.
template <int T, bool OUT>
kq_status launch_side(const OutArgs& oa, int count, hipStream_t st) {
  int nmax = 0;
  bool vec = true;
  for (int l = 0; l < count; ++l) {
    nmax = oa.n[l] > nmax ? oa.n[l] : nmax;
    vec = vec && side_vec_ok(oa.src[l], oa.dst[l], oa.n[l], oa.sd[l]);
  }
  const size_t lds = side_lds_bytes(nmax, T);
  const char* name = OUT ? "decode_out_kernel" : "decode_in_kernel";
  // (the grouped output side holds 16 T values, 16 factors and 16 scales per thread: up to
  // two tokens within the 1024-thread register budget)
  constexpr bool kVecForm = !OUT || T <= 2;
  vec = vec && kVecForm;
  constexpr auto vec_kernel = side_kernel<T, OUT, kVecForm>;  // the scalar form when not allowed
  const void* fn = vec ? reinterpret_cast<const void*>(vec_kernel)
                       : reinterpret_cast<const void*>(&side_kernel<T, OUT, false>);
  if (!allow_lds(fn, lds)) return fail(KQ_EDEVICE, "%s: %zu bytes of LDS refused", name, lds);
  {
    LaunchTimer timer(name, st);
    if (vec)
      hipLaunchKernelGGL(vec_kernel, dim3(count), dim3(kSideThreads), lds, st, oa);
    else
      hipLaunchKernelGGL((side_kernel<T, OUT, false>), dim3(count), dim3(kSideThreads), lds, st, oa);
  }
  return check_launch(name);
}

// in_mode: 0 no input side, 1 fused into the matvec, 2 separate launch into x1.
template <int C, int CPL, int T>
kq_status launch(DecodeArgs a, int in_mode, float* x1, const OutArgs& out, int n_out, hipStream_t st) {
  kq_status s = KQ_OK;
  if (in_mode == 2) {
    OutArgs ia{};
    ia.src[0] = a.x;
    ia.dst[0] = x1;
    ia.n[0] = static_cast<int>(a.din);
    ia.sd[0] = a.in;
    if ((s = launch_side<T, false>(ia, 1, st)) != KQ_OK) return s;
    a.x = x1;
  }
  const Layer& last = a.layer[a.n_layers - 1];
  const unsigned grid = static_cast<unsigned>(last.wg0 + (last.dout + kRowsPerWg - 1) / kRowsPerWg);
  const size_t lds = in_mode == 1 ? side_lds_bytes(a.din, T) : 0;
  const void* fn = in_mode == 1 ? reinterpret_cast<const void*>(&decode_kernel<C, CPL, T, true>)
                                : reinterpret_cast<const void*>(&decode_kernel<C, CPL, T, false>);
  if (!allow_lds(fn, lds)) return fail(KQ_EDEVICE, "decode_kernel: %zu bytes of LDS refused", lds);
  {
    LaunchTimer timer("decode_kernel", st);
    if (in_mode == 1)
      hipLaunchKernelGGL((decode_kernel<C, CPL, T, true>), dim3(grid), dim3(kThreads), lds, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<C, CPL, T, false>), dim3(grid), dim3(kThreads), 0, st, a);
  }
  if ((s = check_launch("decode_kernel")) != KQ_OK || n_out == 0) return s;
  return launch_side<T, true>(out, n_out, st);
}

template <int C>
kq_status launch_t(const DecodeArgs& a, int in_mode, float* x1, const OutArgs& out, int n_out, int cpl,
                   int tokens, hipStream_t st) {
  if (cpl == 16) {
    switch (tokens) {
      case 1: return launch<C, 16, 1>(a, in_mode, x1, out, n_out, st);
      case 2: return launch<C, 16, 2>(a, in_mode, x1, out, n_out, st);
      case 3: return launch<C, 16, 3>(a, in_mode, x1, out, n_out, st);
      default: return launch<C, 16, 4>(a, in_mode, x1, out, n_out, st);
    }
  }
  if (cpl == 32)
    return tokens == 1 ? launch<C, 32, 1>(a, in_mode, x1, out, n_out, st)
                       : launch<C, 32, 2>(a, in_mode, x1, out, n_out, st);
  return launch<C, 64, 1>(a, in_mode, x1, out, n_out, st);
}

size_t y1_bytes(int64_t dout, int64_t tokens) { return align_up(size_t(tokens) * dout * sizeof(float), 256); }

Side make_side(const kq_rot* r, const double* s) {
  Side sd{};
  sd.on = r != nullptr;
  sd.m = 1;
  if (r) {
    sd.m = r->m;
    sd.log2p = r->log2p;
    sd.signs = r->signs;
    sd.q = r->q;
  }
  sd.s = s;
  return sd;
}

}  // namespace

int container_bits(int bits) { return bits == 2 ? 2 : (bits <= 4 ? 4 : 8); }

// dout: the layers' total rows. Each layer's matvec result starts on a 256-byte boundary (the
// padding is covered by one 256-byte slot per layer), then x1.
size_t decode_workspace(int64_t dout, int64_t din, int64_t tokens) {
  return y1_bytes(dout, tokens) + KQ_DECODE_MAX_LAYERS * 256 + align_up(size_t(tokens) * din * sizeof(float), 256);
}

size_t decode_lds_bytes(int64_t dout, int64_t din, int64_t tokens, bool in_side, bool out_rot) {
  const size_t a = in_side ? side_lds_bytes(din, tokens) : 0;
  const size_t b = out_rot ? side_lds_bytes(dout, tokens) : 0;
  return a > b ? a : b;
}

// Codes per lane for a row of din codes with `tokens` tokens: 16, 32 or 64 (the registers
// hold codes-per-lane x tokens <= 64 x1 values), 0 if the shape is out of range.
int decode_cpl(int64_t din, int64_t tokens) {
  for (int cpl = 16; cpl <= 64; cpl *= 2)
    if (din <= int64_t(256) * cpl && cpl * tokens <= 64) return cpl;
  return 0;
}

kq_status pack_run(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint32_t* packed, hipStream_t st) {
  const int c = container_bits(bits);
  const int64_t n = rows * (cols / (32 / c));
  if (n == 0) return KQ_OK;
  {
    LaunchTimer timer("pack_kernel", st);
    hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, codes, rows,
                       cols, c, packed);
  }
  return check_launch("pack_kernel");
}

// Scratch of kq_decode_matvec_group_noalloc: a fixed array of device memory, one copy per GPU,
// held until the process ends. Host code never hands `scratch` itself to a kernel (in host code
// the name stands in for the symbol, not for a device address): its address on the current
// device comes from hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) char scratch[KQ_DECODE_NOALLOC_SCRATCH];

// The largest workspace a valid call can ask for: matvec results of KQ_DECODE_MAX_LAYERS layers
// of KQ_MAX_ROT_DIM rows, their alignment slots, and x1 (din * tokens <= 16384 floats).
static_assert(size_t(KQ_DECODE_MAX_TOKENS) * KQ_DECODE_MAX_LAYERS * KQ_MAX_ROT_DIM * sizeof(float) +
                      KQ_DECODE_MAX_LAYERS * 256 + 16384 * sizeof(float) <=
                  size_t(KQ_DECODE_NOALLOC_SCRATCH),
              "the fixed decode scratch holds every valid call's workspace");

constexpr int kMaxDevices = 64;

kq_status decode_static_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  const hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return fail(KQ_EDEVICE, "decode scratch: hipGetDevice: %s", hipGetErrorString(de));
  if (dev < 0 || dev >= kMaxDevices) return fail(KQ_EUNSUPPORTED, "decode scratch: device %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KQ_EDEVICE, "decode scratch: hipGetSymbolAddress on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return KQ_OK;
}

kq_status decode_run(const kq_decode_layer* layers, int n_layers, int64_t din, int bits, int group,
                     const double* s_x, const kq_rot* rot_in, const float* x, int64_t tokens, void* ws,
                     hipStream_t st) {
  DecodeArgs a{};
  OutArgs out{};
  int n_out = 0, wg = 0;
  int64_t total = 0;
  char* wp = static_cast<char*>(ws);
  for (int l = 0; l < n_layers; ++l) {
    const kq_decode_layer& L = layers[l];
    Layer& d = a.layer[l];
    d.packed = L.packed;
    d.scales = L.scales;
    d.zeros = L.zeros;
    d.dout = L.dout;
    d.y = L.y;
    d.s_g = L.s_g;
    d.wg0 = wg;
    d.y1 = nullptr;
    if (L.rot_out) {
      d.y1 = reinterpret_cast<float*>(wp);
      wp += y1_bytes(L.dout, tokens);
      out.src[n_out] = d.y1;
      out.dst[n_out] = L.y;
      out.n[n_out] = static_cast<int>(L.dout);
      out.sd[n_out] = make_side(L.rot_out, L.s_g);
      ++n_out;
    }
    wg += static_cast<int>((L.dout + kRowsPerWg - 1) / kRowsPerWg);
    total += L.dout;
  }
  a.n_layers = n_layers;
  a.din = din;
  a.group = group;
  a.ngroups = group ? static_cast<int>(din / group) : 1;
  a.x = x;
  a.in = make_side(rot_in, s_x);
  float* x1 = reinterpret_cast<float*>(static_cast<char*>(ws) + y1_bytes(total, tokens) + KQ_DECODE_MAX_LAYERS * 256);
  // The input side runs inside the matvec (in the grouped form) when it is a plain transform (no
  // odd factor), the grid is at most one workgroup per CU (each workgroup repeats it: more would
  // queue the copies behind each other) and its operands are 16-byte aligned; otherwise as its
  // own one-workgroup launch. The direct path reads x as float4s, so an unaligned x with no input
  // side goes through that launch too.
  const bool need_in = rot_in || s_x || !aligned16(x);
  const bool fuse = a.in.m == 1 && wg <= kCus && side_vec_ok(x, nullptr, din, a.in);
  const int in_mode = !need_in ? 0 : (fuse ? 1 : 2);
  const int t = static_cast<int>(tokens);
  const int cpl = decode_cpl(din, tokens);
  switch (container_bits(bits)) {
    case 2: return launch_t<2>(a, in_mode, x1, out, n_out, cpl, t, st);
    case 4: return launch_t<4>(a, in_mode, x1, out, n_out, cpl, t, st);
    default: return launch_t<8>(a, in_mode, x1, out, n_out, cpl, t, st);
  }
}

}  // namespace kq
