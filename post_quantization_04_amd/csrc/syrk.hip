// H = alpha * A^T A + beta * H for token-major bf16 A on gfx950 bf16 MFMA.
//
// A is [rows, d]: tokens by channels, channels contiguous. The contraction
// runs over tokens, so each MFMA operand needs consecutive tokens of one
// channel per lane. Panels of 64 tokens x 256 channels are copied straight
// from global memory into LDS in their natural token-major layout
// (global_load_lds_dwordx4, no register staging), and the MFMA fragments are
// read with the gfx950 transposing LDS load ds_read_b64_tr_b16: in each group
// of 16 lanes, four lanes per token supply 16 consecutive channels and lane j
// receives channel j at the four tokens. Two such loads give the eight tokens
// of a v_mfma_f32_32x32x16_bf16 operand. The 16-byte chunks of each 512-byte
// token row are XOR-swizzled with the token index so that both the DMA writes
// and the transposing reads run at the LDS bank minimum.
//
// LDS holds two stages (2 x 2 panels x 32 KB); the loads of stage s + 1 are in
// flight while the MFMAs of stage s run, with one barrier per stage. A final
// partial stage (fewer than 64 tokens) or a misaligned row pitch takes a
// register path that zero-fills missing tokens.
//
// Work item = (lower-triangle 256 x 256 output tile, token slice of 8192
// rows). Each workgroup sums one slice in float32 MFMA accumulators (bf16
// products are exact) and writes the float32 partial tile. A second kernel
// adds the slices of a tile in float64, applies alpha and beta, rounds once to
// float32 and writes both triangles. Short float32 runs keep the accumulated
// rounding near 1e-7 relative, which the downstream column sweep needs.
//
// Workgroups are dispatched round robin over the 8 XCDs; work items are
// renumbered so that each XCD runs a contiguous run of a blocked tile order
// (4 tile rows x 8 tile columns), whose 32 concurrent workgroups share about
// 12 channel panels in that XCD's L2.
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

typedef short v4i16 __attribute__((ext_vector_type(4)));

#define KQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define KQ_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))

// 16-byte slot of (token t, channel chunk cc) in a panel stage: 32 chunks per
// token row, chunk position XOR 4 * (t mod 4) inside each half row.
__device__ __forceinline__ int slot(int t, int cc) { return t * 32 + ((cc & 16) | ((cc & 15) ^ ((t & 3) << 2))); }

// Triangular tile numbering: t = I (I + 1) / 2 + J with J <= I.
__device__ __forceinline__ void tri(int t, int& I, int& J) {
  int i = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  I = i;
  J = t - i * (i + 1) / 2;
}

// Full stage, aligned rows (lda and d multiples of 8): each wave copies 512
// slots with 8 DMA loads. Lane l of load i fills slot (wave * 512 + i * 64 + l);
// its global chunk is the un-swizzled position. Chunks past channel d re-read
// the row's last 8 channels (their outputs are discarded); every token exists.
__device__ __forceinline__ void load_stage_dma(const uint16_t* __restrict__ a, int64_t lda, int64_t d, int64_t c0,
                                               int64_t t0, uint4* __restrict__ panel) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sl = wave * 512 + i * 64 + lane;
    const int t = sl >> 5, cs = sl & 31;
    const int cc = (cs & 16) | ((cs & 15) ^ ((t & 3) << 2));
    int64_t ch = c0 + int64_t(cc) * 8;
    if (ch > d - 8) ch = d - 8;
    __builtin_amdgcn_global_load_lds(KQ_GLOBAL(a + (t0 + t) * lda + ch), KQ_LDS(panel + wave * 512 + i * 64), 16, 0, 0);
  }
}

// Any stage: register loads with zero fill for tokens >= tok_end and channels >= d.
__device__ __forceinline__ void load_stage_regs(const uint16_t* __restrict__ a, int64_t lda, int64_t d, int64_t c0,
                                                int64_t t0, int64_t tok_end, bool vec_ok, uint4* __restrict__ panel) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sl = i * 256 + static_cast<int>(threadIdx.x);
    const int t = sl >> 5, cs = sl & 31;
    const int cc = (cs & 16) | ((cs & 15) ^ ((t & 3) << 2));
    const int64_t ch = c0 + int64_t(cc) * 8;
    const int64_t tok = t0 + t;
    uint4 val = make_uint4(0, 0, 0, 0);
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
    panel[sl] = val;
  }
}

__device__ __forceinline__ void load_stage(const uint16_t* __restrict__ a, int64_t lda, int64_t d, int64_t c0,
                                           int64_t t0, int64_t tok_end, bool vec_ok, uint4* __restrict__ panel) {
  if (vec_ok && t0 + kKT <= tok_end) load_stage_dma(a, lda, d, c0, t0, panel);
  else load_stage_regs(a, lda, d, c0, t0, tok_end, vec_ok, panel);
}

// MFMA operand: 8 tokens (kk * 16 + 8 (lane / 32) + 0..7) of channel ch0 + lane % 32.
__device__ __forceinline__ bf16x8 frag_tr(const uint4* __restrict__ panel, int ch0, int kk) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int ch = ch0 + 16 * (g & 1) + 4 * (j & 3);
  const int cc = ch >> 3, half = (ch >> 2) & 1;
  const int tb = kk * 16 + 8 * (g >> 1) + (j >> 2);
  const char* base = reinterpret_cast<const char*>(panel) + half * 8;
  const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)KQ_LDS(base + slot(tb, cc) * 16));
  const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)KQ_LDS(base + slot(tb + 4, cc) * 16));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 r = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Lower-triangle tiles in blocks of 4 tile rows x 8 tile columns (row-major
// inside a block): 32 consecutive work items share about 12 channel panels.
__global__ void tile_order_kernel(int nt, int* __restrict__ order) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int r = 0;
  for (int bi = 0; bi < nt; bi += 4)
    for (int bj = 0; bj <= bi + 3 && bj < nt; bj += 8)
      for (int i = bi; i < bi + 4 && i < nt; ++i)
        for (int j = bj; j < bj + 8 && j <= i; ++j) order[r++] = i * (i + 1) / 2 + j;
}

__global__ __launch_bounds__(kThreads, 1) void syrk_partial(
    const uint16_t* __restrict__ a, int64_t lda, int64_t d, int64_t rows, int ntiles, int slice0,
    int nsl, int per_xcd, int vec_ok, const int* __restrict__ order, float* __restrict__ part) {
  __shared__ uint4 lds[2][2][kPanelUnits];  // [stage buffer][panel I, panel J] (128 KB)

  // XCD-aware renumbering: XCD x = blockIdx % 8 takes items [x * per_xcd, (x + 1) * per_xcd).
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= ntiles * nsl) return;
  const int sl = item / ntiles;
  const int tile = order[item - sl * ntiles];
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

  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};

  load_stage(a, lda, d, cI, tok_begin, tok_end, vec_ok, lds[0][0]);
  if (!diag) load_stage(a, lda, d, cJ, tok_begin, tok_end, vec_ok, lds[0][1]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int s = 0; s < nstage; ++s) {
    const int cur = s & 1;
    if (s + 1 < nstage) {
      const int64_t t0 = tok_begin + int64_t(s + 1) * kKT;
      load_stage(a, lda, d, cI, t0, tok_end, vec_ok, lds[cur ^ 1][0]);
      if (!diag) load_stage(a, lda, d, cJ, t0, tok_end, vec_ok, lds[cur ^ 1][1]);
    }
    const uint4* pa = lds[cur][0];
    const uint4* pb = diag ? lds[cur][0] : lds[cur][1];
#pragma unroll
    for (int kk = 0; kk < kKT / 16; ++kk) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) fa[x] = frag_tr(pa, wi * 128 + x * 32, kk);
#pragma unroll
      for (int y = 0; y < 4; ++y) fb[y] = frag_tr(pb, wj * 128 + y * 32, kk);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
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
  size_t part_bytes, acc_bytes, order_bytes;
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
  p.order_bytes = align_up(size_t(p.ntiles) * sizeof(int), 256);
  return p;
}

}  // namespace

size_t syrk_workspace(int64_t rows, int64_t d) {
  if (rows <= 0) return 0;
  const Plan p = plan(rows, d);
  return p.part_bytes + p.acc_bytes + p.order_bytes;
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
  int* order = reinterpret_cast<int*>(static_cast<char*>(ws) + p.part_bytes + p.acc_bytes);
  // 16-byte loads need aligned rows; the DMA path also needs whole 8-channel chunks
  const int vec_ok = (lda % 8 == 0) && (d % 8 == 0) && (reinterpret_cast<uintptr_t>(a) % 16 == 0);
  {
    LaunchTimer timer("tile_order_kernel", st);
    hipLaunchKernelGGL(tile_order_kernel, dim3(1), dim3(64), 0, st, p.nt, order);
  }
  kq_status s0 = check_launch("tile_order_kernel");
  if (s0 != KQ_OK) return s0;
  for (int g = 0; g < p.ngroups; ++g) {
    const int s0 = g * p.group;
    const int nsl = (s0 + p.group <= p.nslices) ? p.group : p.nslices - s0;
    const int items = p.ntiles * nsl;
    const int per_xcd = (items + kXcds - 1) / kXcds;
    {
      LaunchTimer timer("syrk_partial", st);
      hipLaunchKernelGGL(syrk_partial, dim3(static_cast<unsigned>(per_xcd * kXcds)), dim3(kThreads), 0, st, a,
                         lda, d, rows, p.ntiles, s0, nsl, per_xcd, vec_ok, order, part);
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
