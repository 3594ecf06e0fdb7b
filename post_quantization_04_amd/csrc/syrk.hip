// H = alpha * A^T A + beta * H for token-major bf16 A on gfx950 bf16 MFMA.
//
// A is [rows, d]: tokens by channels, channels contiguous. The contraction
// runs over tokens, so each MFMA operand needs eight consecutive tokens of one
// channel per lane. A thread loads an 8 token x 8 channel block with eight
// 16-byte global loads (coalesced along channels), transposes it in registers
// with 16-bit shuffles and writes eight channel-major 16-byte packs to LDS.
// MFMA fragments are then single ds_read_b128 loads. LDS rows are 128 bytes
// (64 tokens) and the 16-byte chunks of a row are XOR-swizzled with the row
// index so that both the transposing writes and the fragment reads are free of
// bank conflicts.
//
// Work item = (lower-triangle 256 x 256 output tile, token slice of 8192
// rows). Each workgroup sums one slice in float32 MFMA accumulators
// (v_mfma_f32_32x32x16_bf16; bf16 products are exact) and writes the float32
// partial tile. A second kernel adds the slices of a tile in float64, applies
// alpha and beta, rounds once to float32 and writes both triangles. Short
// float32 runs keep the accumulated rounding near 1e-7 relative, which the
// downstream column sweep needs.
//
// Workgroups are dispatched round robin over the 8 XCDs; work items are
// renumbered so that each XCD takes a contiguous run of tiles of one slice,
// which share their channel panels in that XCD's L2.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kT = 256;          // output tile edge (channels)
constexpr int kKT = 64;          // tokens per LDS stage
constexpr int kSlice = 8192;     // tokens per float32 partial sum
constexpr int kThreads = 256;    // 4 waves in a 2 x 2 grid, 128 x 128 outputs each
constexpr int kPanelUnits = kT * kKT * 2 / 16;  // 16-byte units per LDS panel (2048)
constexpr int kTargetItems = 2048;  // work items per launch before slices are split into groups

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16-byte unit index of (channel row, token chunk) in a panel.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 8 + (chunk ^ ((row & 7) ^ ((row >> 3) & 7)));
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Triangular tile numbering: t = I (I + 1) / 2 + J with J <= I.
__device__ __forceinline__ void tri(int t, int& I, int& J) {
  int i = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  I = i;
  J = t - i * (i + 1) / 2;
}

// Global loads of one 8 x 8 block of the thread: rows tok0 + 8 tg + r, channels c0 + 8 cg ...
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ a, int64_t lda, int64_t d,
                                           int64_t c0, int64_t tok0, int64_t tok_end, bool vec_ok,
                                           uint4 (&v)[8]) {
  const int tid = threadIdx.x;
  const int64_t ch = c0 + (tid & 31) * 8;
  const int64_t tb = tok0 + (tid >> 5) * 8;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint4 val = make_uint4(0, 0, 0, 0);
    const int64_t tok = tb + r;
    if (tok < tok_end && ch < d) {
      const uint16_t* p = a + tok * lda + ch;
      if (vec_ok && ch + 8 <= d) {
        val = *reinterpret_cast<const uint4*>(p);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = (ch + k < d) ? p[k] : uint16_t(0);
        val.x = e[0] | (uint32_t(e[1]) << 16);
        val.y = e[2] | (uint32_t(e[3]) << 16);
        val.z = e[4] | (uint32_t(e[5]) << 16);
        val.w = e[6] | (uint32_t(e[7]) << 16);
      }
    }
    v[r] = val;
  }
}

// Transpose the 8 x 8 block (tokens x channels) and store channel-major packs.
__device__ __forceinline__ void store_block(uint4* __restrict__ panel, const uint4 (&v)[8]) {
  const int tid = threadIdx.x;
  const int cg = tid & 31, tg = tid >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t out[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = word(v[2 * k], c >> 1);
      const uint32_t hi = word(v[2 * k + 1], c >> 1);
      out[k] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    panel[swz(cg * 8 + c, tg)] = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

__device__ __forceinline__ bf16x8 frag(const uint4* __restrict__ panel, int row, int chunk) {
  return __builtin_bit_cast(bf16x8, panel[swz(row, chunk)]);
}

__global__ __launch_bounds__(kThreads, 1) void syrk_partial(
    const uint16_t* __restrict__ a, int64_t lda, int64_t d, int64_t rows, int ntiles, int slice0,
    int nsl, int per_xcd, int vec_ok, float* __restrict__ part) {
  __shared__ uint4 lds[2][kPanelUnits];  // panel I, panel J (64 KB)

  // XCD-aware renumbering: XCD x = blockIdx % 8 takes items [x * per_xcd, (x + 1) * per_xcd).
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= ntiles * nsl) return;
  const int sl = item / ntiles;
  const int tile = item - sl * ntiles;
  int I, J;
  tri(tile, I, J);
  const bool diag = (I == J);
  const int64_t cI = int64_t(I) * kT, cJ = int64_t(J) * kT;
  const int64_t tok_begin = int64_t(slice0 + sl) * kSlice;
  const int64_t tok_end = tok_begin + kSlice < rows ? tok_begin + kSlice : rows;
  const int nstage = static_cast<int>((tok_end - tok_begin + kKT - 1) / kKT);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const uint4* pa = lds[0];
  const uint4* pb = diag ? lds[0] : lds[1];

  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};

  uint4 va[8], vb[8];
  load_block(a, lda, d, cI, tok_begin, tok_end, vec_ok, va);
  if (!diag) load_block(a, lda, d, cJ, tok_begin, tok_end, vec_ok, vb);

  for (int s = 0; s < nstage; ++s) {
    store_block(lds[0], va);
    if (!diag) store_block(lds[1], vb);
    __syncthreads();
    if (s + 1 < nstage) {
      const int64_t t0 = tok_begin + int64_t(s + 1) * kKT;
      load_block(a, lda, d, cI, t0, tok_end, vec_ok, va);
      if (!diag) load_block(a, lda, d, cJ, t0, tok_end, vec_ok, vb);
    }
#pragma unroll
    for (int kk = 0; kk < kKT / 16; ++kk) {
      const int chunk = 2 * kk + (lane >> 5);
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) fa[x] = frag(pa, wi * 128 + x * 32 + (lane & 31), chunk);
#pragma unroll
      for (int y = 0; y < 4; ++y) fb[y] = frag(pb, wj * 128 + y * 32 + (lane & 31), chunk);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    __syncthreads();
  }

  // D[i][j] of a 32 x 32 block: lane l, register r -> i = 8 (r / 4) + 4 (l / 32) + r % 4, j = l % 32.
  float* out = part + (int64_t(sl) * ntiles + tile) * (kT * kT);
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = wi * 128 + x * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int j = wj * 128 + y * 32 + (lane & 31);
        out[i * kT + j] = acc[x][y][r];
      }
}

// Sums the float32 partials of a tile in float64; at the last slice group
// writes H = alpha * S + beta * H to both triangles (64 x 64 sub-blocks).
__global__ __launch_bounds__(256) void syrk_reduce(const float* __restrict__ part, int nsl, int ntiles,
                                                   int64_t d, double* __restrict__ acc, int first,
                                                   int last, float alpha, float beta,
                                                   float* __restrict__ h) {
  __shared__ float tr[64][65];
  const int tile = blockIdx.x >> 4;
  const int si = (blockIdx.x >> 2) & 3, sj = blockIdx.x & 3;
  int I, J;
  tri(tile, I, J);
  const bool dsub = (I == J) && (si == sj);  // sub-block on the diagonal of H
  if (I == J && sj > si) return;              // mirror of another sub-block
  const int64_t r0 = int64_t(I) * kT + si * 64, c0 = int64_t(J) * kT + sj * 64;
  const int jl = threadIdx.x & 63;
  const int ib = (threadIdx.x >> 6) * 16;
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {
    const int il = ib + k;
    const int64_t e = int64_t(si * 64 + il) * kT + sj * 64 + jl;
    double s = first ? 0.0 : acc[int64_t(tile) * kT * kT + e];
    for (int q = 0; q < nsl; ++q) s += static_cast<double>(part[(int64_t(q) * ntiles + tile) * kT * kT + e]);
    if (!last) {
      acc[int64_t(tile) * kT * kT + e] = s;
    } else {
      const int64_t gi = r0 + il, gj = c0 + jl;
      double v = static_cast<double>(alpha) * s;
      if (beta != 0.0f && gi < d && gj < d && (!dsub || il >= jl))
        v += static_cast<double>(beta) * static_cast<double>(h[gi * d + gj]);
      tr[il][jl] = static_cast<float>(v);
    }
  }
  if (!last) return;
  __syncthreads();
  // lower-triangle position (row-major, coalesced along j)
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {
    const int il = ib + k;
    const int64_t gi = r0 + il, gj = c0 + jl;
    if (gi < d && gj < d && (!dsub || il >= jl)) h[gi * d + gj] = tr[il][jl];
  }
  // mirrored position: H[c0 + a][r0 + b] = S[b][a]
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {
    const int al = ib + k;  // row offset in the mirror block (from the column side)
    const int bl = jl;      // column offset (from the row side)
    const int64_t gi = c0 + al, gj = r0 + bl;
    if (gi < d && gj < d && (!dsub || bl > al)) h[gi * d + gj] = tr[bl][al];
  }
}

__global__ void scale_kernel(float* __restrict__ h, int64_t n, float beta) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) h[i] = (beta == 0.0f) ? 0.0f : beta * h[i];
}

struct Plan {
  int nt, ntiles, nslices, group, ngroups;
  size_t part_bytes, acc_bytes;
};

Plan plan(int64_t rows, int64_t d) {
  Plan p{};
  p.nt = static_cast<int>((d + kT - 1) / kT);
  p.ntiles = p.nt * (p.nt + 1) / 2;
  p.nslices = static_cast<int>((rows + kSlice - 1) / kSlice);
  int g = (kTargetItems + p.ntiles - 1) / p.ntiles;
  if (g < 1) g = 1;
  if (g > p.nslices) g = p.nslices;
  p.group = g;
  p.ngroups = p.nslices ? (p.nslices + g - 1) / g : 0;
  p.part_bytes = align_up(size_t(g) * p.ntiles * kT * kT * sizeof(float), 256);
  p.acc_bytes = p.ngroups > 1 ? align_up(size_t(p.ntiles) * kT * kT * sizeof(double), 256) : 0;
  return p;
}

}  // namespace

size_t syrk_workspace(int64_t rows, int64_t d) {
  if (rows <= 0) return 0;
  const Plan p = plan(rows, d);
  return p.part_bytes + p.acc_bytes;
}

kq_status syrk_run(const uint16_t* a, int64_t rows, int64_t d, int64_t lda, float alpha, float beta,
                   float* h, void* ws, hipStream_t st) {
  if (rows == 0) {
    const int64_t n = d * d;
    {
      LaunchTimer timer("scale_kernel", st);
      hipLaunchKernelGGL(scale_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, h, n,
                         beta);
    }
    return check_launch("scale_kernel");
  }
  const Plan p = plan(rows, d);
  float* part = static_cast<float*>(ws);
  double* acc = reinterpret_cast<double*>(static_cast<char*>(ws) + p.part_bytes);
  const int vec_ok = (lda % 8 == 0) && (reinterpret_cast<uintptr_t>(a) % 16 == 0);
  for (int g = 0; g < p.ngroups; ++g) {
    const int s0 = g * p.group;
    const int nsl = (s0 + p.group <= p.nslices) ? p.group : p.nslices - s0;
    const int items = p.ntiles * nsl;
    const int per_xcd = (items + kXcds - 1) / kXcds;
    {
      LaunchTimer timer("syrk_partial", st);
      hipLaunchKernelGGL(syrk_partial, dim3(static_cast<unsigned>(per_xcd * kXcds)), dim3(kThreads), 0, st, a,
                         lda, d, rows, p.ntiles, s0, nsl, per_xcd, vec_ok, part);
    }
    kq_status s = check_launch("syrk_partial");
    if (s != KQ_OK) return s;
    {
      LaunchTimer timer("syrk_reduce", st);
      hipLaunchKernelGGL(syrk_reduce, dim3(static_cast<unsigned>(p.ntiles * 16)), dim3(256), 0, st, part, nsl,
                         p.ntiles, d, acc, g == 0 ? 1 : 0, g == p.ngroups - 1 ? 1 : 0, alpha, beta, h);
    }
    s = check_launch("syrk_reduce");
    if (s != KQ_OK) return s;
  }
  return KQ_OK;
}

}  // namespace kq
