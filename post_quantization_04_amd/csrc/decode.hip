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
// Per layer and token batch (T <= 4 tokens):
//   1. every workgroup forms x1 = U_X S_X^-1 x in LDS (signs and scales on
//      load, fast Walsh-Hadamard transform per 2^k chunk in radix-16 register
//      passes, odd-factor mix across the m chunks) and keeps the entries its
//      lanes need in registers;
//   2. 16 rows per workgroup: the four waves split each row's packed words
//      (lane l of wave w reads word 64 w + l + 256 i), dequantize on the fly,
//      y1[row] = sum_g s_g (sum_j q_j x1_j - z_g sum_j x1_j), one 32-bit load
//      per word and row, the loads of all 16 rows in flight at once for
//      rows of up to 256 words;
//   3. a second, one-workgroup launch applies the output side to y1:
//      transform per chunk, transposed odd mix, signs, 1 / s_g. (A fused
//      last-workgroup variant needed a device-scope fence in every workgroup,
//      which cost more than the launch.)
// Everything is float32; the float64 diagonal scales and rotation factors are
// rounded to float32 on load.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWg = 16;
constexpr int kBatch = 8;  // vector entries per thread whose loads are issued together

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

struct DecodeArgs {
  const uint32_t* packed;
  const float* scales;
  const uint8_t* zeros;
  int64_t dout, din;
  int group, ngroups;
  Side in, out;
  const float* x;   // [T, din]
  float* y;         // [T, dout]
  float* y1;        // scratch [T, dout]
};

// One pass of the fast Walsh-Hadamard transform over index bits [o, o + R) of every token's
// n entries (pitch n): a thread owns the 2^R entries of one group (indices that differ only in
// those bits) and does the R butterfly stages in registers.
template <int T, int R>
__device__ void fwht_pass(float* v, int n, int o) {
  constexpr int L = 1 << R;
  const int groups = n >> R, stride = 1 << o;
  for (int e = threadIdx.x; e < T * groups; e += kThreads) {
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

// H_p (unnormalised) on every chunk of p = 2^log2p entries of each token's n = m p entries.
template <int T>
__device__ void fwht_lds(float* v, int n, int log2p) {
  for (int o = 0; o < log2p; o += 4) {
    switch (log2p - o) {
      case 1: fwht_pass<T, 1>(v, n, o); break;
      case 2: fwht_pass<T, 2>(v, n, o); break;
      case 3: fwht_pass<T, 3>(v, n, o); break;
      default: fwht_pass<T, 4>(v, n, o); break;
    }
  }
}

// Odd-factor mix across the m chunks of p (column b of the m x p view of each token's
// vector): out[a] = sum_a' W[a][a'] v[a'] with W = Q (TRANS: Q^T), times `post`
// (1 / sqrt(p)). W is staged in LDS as float32 with qs[a' * 64 + a] = W[a][a'] post; a
// thread forms the m outputs of one column 16 at a time, reading the 16 weights of each
// input as four workgroup-uniform float4s. OOP: the outputs go to dst (same layout as v)
// as they are formed; otherwise they go back to v once all of the column's are formed.
constexpr int kQPitch = 64;  // (e >> 6 and e & 63 below rely on it)
template <int T, bool TRANS, bool OOP>
__device__ void mix_lds(float* v, float* dst, int n, int m, int log2p, const double* __restrict__ q, float* qs,
                        float post) {
  // batches of kBatch entries per thread, every load issued before the stores
  for (int base = 0; base < m * kQPitch; base += kBatch * kThreads) {
    float qb[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = base + k * kThreads + static_cast<int>(threadIdx.x);
      const int a2 = e >> 6, a = e & (kQPitch - 1);
      qb[k] = (e < m * kQPitch && a < m) ? static_cast<float>(TRANS ? q[a2 * m + a] : q[a * m + a2]) * post : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = base + k * kThreads + static_cast<int>(threadIdx.x);
      if (e < m * kQPitch) qs[e] = qb[k];
    }
  }
  __syncthreads();
  const int p = 1 << log2p;
  if constexpr (OOP) {
    for (int e = threadIdx.x; e < T * p; e += kThreads) {
      const int t = e >> log2p, b = e & (p - 1);
      const float* row = v + t * n + b;
      float* out = dst + t * n + b;
      for (int ag = 0; ag < m; ag += 16) {
        float acc[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
        for (int a2 = 0; a2 < m; ++a2) {
          const float x = row[a2 * p];
          const float4* w = reinterpret_cast<const float4*>(qs + a2 * kQPitch + ag);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float4 wc = w[c];
            acc[4 * c] = fmaf(wc.x, x, acc[4 * c]);
            acc[4 * c + 1] = fmaf(wc.y, x, acc[4 * c + 1]);
            acc[4 * c + 2] = fmaf(wc.z, x, acc[4 * c + 2]);
            acc[4 * c + 3] = fmaf(wc.w, x, acc[4 * c + 3]);
          }
        }
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (ag + k < m) out[(ag + k) * p] = acc[k];
      }
    }
    __syncthreads();
    return;
  }
  for (int e = threadIdx.x; e < T * p; e += kThreads) {
    const int t = e >> log2p, b = e & (p - 1);
    float* row = v + t * n + b;
    // the group loop is unrolled, so every index into res is a constant (registers only); the
    // column's inputs stay in LDS until all its outputs are formed
    constexpr int kGroups = (KQ_MAX_ODD + 15) / 16;
    float res[kGroups][16];
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
#pragma unroll
      for (int k = 0; k < 16; ++k) res[gi][k] = 0.0f;
      if (16 * gi < m) {
        for (int a2 = 0; a2 < m; ++a2) {
          const float x = row[a2 * p];
          const float4* w = reinterpret_cast<const float4*>(qs + a2 * kQPitch + 16 * gi);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float4 wc = w[c];
            res[gi][4 * c] = fmaf(wc.x, x, res[gi][4 * c]);
            res[gi][4 * c + 1] = fmaf(wc.y, x, res[gi][4 * c + 1]);
            res[gi][4 * c + 2] = fmaf(wc.z, x, res[gi][4 * c + 2]);
            res[gi][4 * c + 3] = fmaf(wc.w, x, res[gi][4 * c + 3]);
          }
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi)
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (16 * gi + k < m) row[(16 * gi + k) * p] = res[gi][k];
  }
  __syncthreads();
}

// Code k (k < 32 / C) of a packed word with C-bit containers, as a float.
template <int C>
__device__ __forceinline__ float code_at(uint32_t w, int k) {
  return static_cast<float>((w >> (C * k)) & ((1u << C) - 1u));
}

// Floats at the front of the matvec kernel's LDS: the T x1 vectors, later the row partials.
__host__ __device__ constexpr int main_vec_floats(int din, int tokens) {
  return tokens * din > kRowsPerWg * 4 * tokens ? tokens * din : kRowsPerWg * 4 * tokens;
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
// their x1 values; T: tokens (CPL T <= 64).
template <int C, int CPL, int T>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs g) {
  extern __shared__ float lds[];
  constexpr int PER = 32 / C;          // codes per word
  constexpr int NW = CPL / PER;        // words per lane per row
  constexpr int U = NW == 1 ? 16 : (NW == 2 ? 8 : (NW == 4 ? 2 : 1));  // rows in flight
  static_assert(NW >= 1 && CPL % PER == 0, "codes per lane");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t din = g.din, dout = g.dout;
  const int64_t wpr = din / PER;  // words per row

  // the first rows' codes, scales and zero points do not depend on x: their loads go first
  const int64_t r0 = int64_t(blockIdx.x) * kRowsPerWg;
  uint32_t wd[U][NW];
  float sc[U][NW], ze[U][NW];
  auto load_rows = [&](int rb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + rb + u;
      const bool rv = row < dout;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const int64_t k = 64 * wave + lane + 256 * i;
        const bool ok = rv && k < wpr;
        wd[u][i] = ok ? g.packed[row * wpr + k] : 0u;
        const int64_t gi = g.group ? (k * PER) / g.group : 0;
        sc[u][i] = ok ? g.scales[row * g.ngroups + gi] : 0.0f;
        ze[u][i] = ok ? static_cast<float>(g.zeros[row * g.ngroups + gi]) : 0.0f;
      }
    }
  };
  load_rows(0);

  // 1. x1 = U_X S_X^-1 x, in LDS [T][din]; Q of a mixed side staged after the vectors, the
  // mixed vectors after Q
  const int din32 = static_cast<int>(din);
  float* qs = lds + main_vec_floats(din32, T);
  float* mixed = qs + KQ_MAX_ODD * kQPitch;
  const float post_in = g.in.on ? 1.0f / sqrtf(static_cast<float>(1 << g.in.log2p)) : 1.0f;
  // batches of kBatch entries per thread: every load of a batch is issued before its stores
  for (int base = 0; base < din32; base += kBatch * kThreads) {
    float xb[kBatch][T], fb[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int j = base + k * kThreads + tid;
      const bool ok = j < din32;
      const float sg = (ok && g.in.on && g.in.signs[j] < 0) ? -1.0f : 1.0f;
      fb[k] = (ok && g.in.s) ? sg / static_cast<float>(g.in.s[j]) : sg;
#pragma unroll
      for (int t = 0; t < T; ++t) xb[k][t] = ok ? g.x[t * din + j] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int j = base + k * kThreads + tid;
      if (j < din32) {
#pragma unroll
        for (int t = 0; t < T; ++t) lds[t * din32 + j] = xb[k][t] * fb[k];
      }
    }
  }
  __syncthreads();
  const float* x1 = lds;
  if (g.in.on) {
    fwht_lds<T>(lds, din32, g.in.log2p);
    if (g.in.m > 1) {
      mix_lds<T, false, true>(lds, mixed, din32, g.in.m, g.in.log2p, g.in.q, qs, post_in);
      x1 = mixed;
    }
  }
  const float xscale = (g.in.on && g.in.m == 1) ? post_in : 1.0f;
  // this lane's words: k = 64 wave + lane + 256 i
  float xv[NW][PER][T];
  float xs[NW][T];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int64_t k = 64 * wave + lane + 256 * i;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float sum = 0.0f;
#pragma unroll
      for (int c = 0; c < PER; ++c) {
        const float v = k < wpr ? x1[t * din32 + static_cast<int>(k) * PER + c] * xscale : 0.0f;
        xv[i][c][t] = v;
        sum += v;
      }
      xs[i][t] = sum;
    }
  }
  __syncthreads();  // LDS is reused for the row partials below

  // 2. rows r0 .. r0 + 15: partial sums per wave, U rows at a time
  float* part = lds;  // [kRowsPerWg][4][T]
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
          acc[t] = fmaf(sc[u][i], fmaf(-ze[u][i], xs[i][t], dot), acc[t]);
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
  const bool rotate_out = g.out.on != 0;
  for (int e = tid; e < kRowsPerWg * T; e += kThreads) {
    const int rr = e / T, t = e % T;
    const int64_t row = r0 + rr;
    if (row >= dout) continue;
    const float* pp = part + rr * 4 * T + t;
    const float v = (pp[0] + pp[T]) + (pp[2 * T] + pp[3 * T]);
    if (rotate_out) {
      g.y1[t * dout + row] = v;
    } else {
      g.y[t * dout + row] = g.out.s ? v / static_cast<float>(g.out.s[row]) : v;
    }
  }
}

// Output side, one workgroup for all tokens: y = S_G^-1 U_G^T y1 (transform per chunk,
// transposed odd mix, signs, 1 / s_g).
template <int T>
__global__ __launch_bounds__(kThreads) void decode_out_kernel(DecodeArgs g) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int dout32 = static_cast<int>(g.dout);
  float* qs = lds + T * dout32;
  for (int base = 0; base < T * dout32; base += kBatch * kThreads) {
    float vb[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = base + k * kThreads + tid;
      vb[k] = e < T * dout32 ? g.y1[e] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = base + k * kThreads + tid;
      if (e < T * dout32) lds[e] = vb[k];
    }
  }
  __syncthreads();
  const float post_out = 1.0f / sqrtf(static_cast<float>(1 << g.out.log2p));
  fwht_lds<T>(lds, dout32, g.out.log2p);
  if (g.out.m > 1) mix_lds<T, true, false>(lds, nullptr, dout32, g.out.m, g.out.log2p, g.out.q, qs, post_out);
  const float yscale = g.out.m > 1 ? 1.0f : post_out;
  for (int base = 0; base < dout32; base += kBatch * kThreads) {
    float fb[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = base + k * kThreads + tid;
      const bool ok = i < dout32;
      const float sg = (ok && g.out.signs[i] < 0) ? -yscale : yscale;
      fb[k] = (ok && g.out.s) ? sg / static_cast<float>(g.out.s[i]) : sg;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = base + k * kThreads + tid;
      if (i < dout32) {
#pragma unroll
        for (int t = 0; t < T; ++t) g.y[t * g.dout + i] = lds[t * dout32 + i] * fb[k];
      }
    }
  }
}

size_t main_lds_bytes(int64_t din, int64_t tokens, bool in_mix) {
  const int64_t f = main_vec_floats(static_cast<int>(din), static_cast<int>(tokens)) + KQ_MAX_ODD * kQPitch +
                    (in_mix ? tokens * din : 0);
  return size_t(f) * sizeof(float);
}

size_t out_lds_bytes(int64_t dout, int64_t tokens) {
  return size_t(tokens * dout + KQ_MAX_ODD * kQPitch) * sizeof(float);
}

bool allow_lds(const void* fn, size_t bytes) {
  return bytes <= 64 * 1024 ||
         hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes)) == hipSuccess;
}

template <int C, int CPL, int T>
kq_status launch(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((a.dout + kRowsPerWg - 1) / kRowsPerWg);
  const size_t lds_main = main_lds_bytes(a.din, T, a.in.on && a.in.m > 1);
  if (!allow_lds(reinterpret_cast<const void*>(&decode_kernel<C, CPL, T>), lds_main))
    return fail(KQ_EDEVICE, "decode_kernel: %zu bytes of LDS refused", lds_main);
  {
    LaunchTimer timer("decode_kernel", st);
    hipLaunchKernelGGL((decode_kernel<C, CPL, T>), dim3(grid), dim3(kThreads), lds_main, st, a);
  }
  kq_status s = check_launch("decode_kernel");
  if (s != KQ_OK || !a.out.on) return s;
  const size_t lds_out = out_lds_bytes(a.dout, T);
  if (!allow_lds(reinterpret_cast<const void*>(&decode_out_kernel<T>), lds_out))
    return fail(KQ_EDEVICE, "decode_out_kernel: %zu bytes of LDS refused", lds_out);
  {
    LaunchTimer timer("decode_out_kernel", st);
    hipLaunchKernelGGL((decode_out_kernel<T>), dim3(1), dim3(kThreads), lds_out, st, a);
  }
  return check_launch("decode_out_kernel");
}

template <int C>
kq_status launch_t(const DecodeArgs& a, int cpl, int tokens, hipStream_t st) {
  if (cpl == 16) {
    switch (tokens) {
      case 1: return launch<C, 16, 1>(a, st);
      case 2: return launch<C, 16, 2>(a, st);
      case 3: return launch<C, 16, 3>(a, st);
      default: return launch<C, 16, 4>(a, st);
    }
  }
  if (cpl == 32) return tokens == 1 ? launch<C, 32, 1>(a, st) : launch<C, 32, 2>(a, st);
  return launch<C, 64, 1>(a, st);
}

Side make_side(const kq_rot* r, const double* s) {
  Side sd{};
  sd.on = r != nullptr;
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

size_t decode_workspace(int64_t dout, int64_t tokens) { return align_up(size_t(tokens) * dout * sizeof(float), 256); }

size_t decode_lds_bytes(int64_t dout, int64_t din, int64_t tokens, bool in_mix, bool out_rot) {
  const size_t a = main_lds_bytes(din, tokens, in_mix);
  const size_t b = out_rot ? out_lds_bytes(dout, tokens) : 0;
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

kq_status decode_run(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t dout, int64_t din,
                     int bits, int group, const double* s_x, const double* s_g, const kq_rot* rot_in,
                     const kq_rot* rot_out, const float* x, int64_t tokens, float* y, void* ws, hipStream_t st) {
  DecodeArgs a{};
  a.packed = packed;
  a.scales = scales;
  a.zeros = zeros;
  a.dout = dout;
  a.din = din;
  a.group = group;
  a.ngroups = group ? static_cast<int>(din / group) : 1;
  a.in = make_side(rot_in, s_x);
  a.out = make_side(rot_out, s_g);
  a.x = x;
  a.y = y;
  a.y1 = static_cast<float*>(ws);
  const int t = static_cast<int>(tokens);
  const int cpl = decode_cpl(din, tokens);
  switch (container_bits(bits)) {
    case 2: return launch_t<2>(a, cpl, t, st);
    case 4: return launch_t<4>(a, cpl, t, st);
    default: return launch_t<8>(a, cpl, t, st);
  }
}

}  // namespace kq
