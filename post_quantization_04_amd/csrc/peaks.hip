// Peak probes for gfx950: sustained matrix-core rates and HBM copy bandwidth
// measured on the machine, as context for the rooflines of the path's kernels
// (which are priced against the published peaks). Not part of the
// quantization path; built into a library of its own.
//
// MFMA probes: 4 waves per workgroup, 4 workgroups per CU, each wave runs
// `iters` rounds of 16 independent MFMAs (a 4 x 4 grid of accumulators over
// four A and four B operand registers) with no memory traffic but one store
// per lane at the end. Operands are either random (hashed from the lane, so
// every MFMA multiplies different, full-entropy values, as the path's kernels
// do) or one constant value (the bits never toggle: the rate the pipes reach
// when power is not the limit). Lane 0 of workgroup 0 reads the shader clock
// counter (s_memtime) and the 100 MHz real-time counter (s_memrealtime) around
// its loop, which gives the clock the loop ran at.
//
// Copy probe: grid-stride copy of 16-byte words, src -> dst, four loads in flight per
// lane, non-temporal (the data is touched once).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kq_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// A value in (-1, 1) from a hash (RANDOM) or 0.5 (constant).
template <bool RANDOM>
__device__ __forceinline__ float operand(uint32_t key) {
  if constexpr (!RANDOM) return 0.5f;
  const uint32_t h = mix(key);
  return static_cast<float>((h & 0xffffu) + (h >> 16)) * (1.0f / 65536.0f) - 1.0f;
}

__device__ __forceinline__ void clock_mark(long long* clk, long long t, long long r, int slot) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    clk[2 * slot] = t;
    clk[2 * slot + 1] = r;
  }
}

template <bool RANDOM>
__global__ __launch_bounds__(256) void bf16_probe(int iters, float* out, long long* clk) {
  const uint32_t key = (blockIdx.x * 256u + threadIdx.x) * 64u;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[x][e] = static_cast<__bf16>(operand<RANDOM>(key + 8 * x + e));
      b[x][e] = static_cast<__bf16>(operand<RANDOM>(key + 32 + 8 * x + e));
    }
  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};
  clock_mark(clk, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime(), 0);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
  clock_mark(clk, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime(), 1);
  float s = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[x][y][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <bool RANDOM>
__global__ __launch_bounds__(256) void f32_probe(int iters, float* out, long long* clk) {
  const uint32_t key = (blockIdx.x * 256u + threadIdx.x) * 64u;
  float a[4], b[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    a[x] = operand<RANDOM>(key + x);
    b[x] = operand<RANDOM>(key + 32 + x);
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};
  clock_mark(clk, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime(), 0);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x], b[y], acc[x][y], 0, 0, 0);
  clock_mark(clk, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime(), 1);
  float s = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[x][y][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// The compiler keeps the loop-carried float64 accumulators in VGPRs and moves
// them through AGPRs around every loop iteration, which drains the MFMA pipe:
// one iteration runs 8 rounds (iters is rounded down to a multiple of 8) so
// the drain is paid once per 128 MFMAs.
template <bool RANDOM>
__global__ __launch_bounds__(256) void f64_probe(int iters, float* out, long long* clk) {
  const uint32_t key = (blockIdx.x * 256u + threadIdx.x) * 64u;
  double a[2], b[4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
    a[x] = static_cast<double>(operand<RANDOM>(key + x)) + 1e-9 * static_cast<double>(operand<RANDOM>(key + 8 + x));
#pragma unroll
  for (int y = 0; y < 4; ++y)
    b[y] = static_cast<double>(operand<RANDOM>(key + 32 + y)) +
           1e-9 * static_cast<double>(operand<RANDOM>(key + 40 + y));
  f64x4 acc[2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f64x4{};
  clock_mark(clk, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime(), 0);
  for (int it = 0; it + 8 <= iters; it += 8)
#pragma unroll
    for (int h = 0; h < 16; ++h)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], b[y], acc[x][y], 0, 0, 0);
  clock_mark(clk, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime(), 1);
  double s = 0.0;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) s += acc[x][y][r];
  out[blockIdx.x * 256 + threadIdx.x] = static_cast<float>(s);
}

// Each thread moves four 16-byte words per round (all four loads issued before the first
// store); consecutive lanes take consecutive words. n is a multiple of 4 * 256.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void copy_probe(const f32x4* __restrict__ src, f32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * 1024;
  for (int64_t base = int64_t(blockIdx.x) * 1024 + threadIdx.x; base < n; base += stride) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + base + 256 * u);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + base + 256 * u);
  }
}

}  // namespace

extern "C" {

// Workgroups of one MFMA probe launch (4 per CU on 256 CUs); `out` must hold
// kqp_mfma_blocks() * 256 floats.
int kqp_mfma_blocks(void) { return 1024; }

// Flops of one wave-round (16 MFMAs) of probe `kind` (float64: iters is rounded down to a
// multiple of 8 rounds).
double kqp_flops_per_round(int kind) {
  switch (kind) {
    case 0:
    case 1: return 16.0 * 32 * 32 * 16 * 2;  // v_mfma_f32_32x32x16_bf16
    case 2:
    case 3: return 16.0 * 32 * 32 * 2 * 2;   // v_mfma_f32_32x32x2f32
    case 4:
    case 5: return 16.0 * 16 * 16 * 4 * 2;   // v_mfma_f64_16x16x4f64
    default: return 0.0;
  }
}

// Launches MFMA probe `kind` on `stream`: 0 bf16 random, 1 bf16 constant, 2 f32 random,
// 3 f32 constant, 4 f64 random, 5 f64 constant. `clk` (device, 4 long longs) receives the
// shader-clock and real-time counters before and after workgroup 0's loop.
// Returns 0, or -1 for an unknown kind or bad arguments.
int kqp_mfma(int kind, int iters, float* out, long long* clk, void* stream) {
  if (iters <= 0 || out == nullptr || clk == nullptr) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(kqp_mfma_blocks()), block(256);
  switch (kind) {
    case 0: hipLaunchKernelGGL(bf16_probe<true>, grid, block, 0, st, iters, out, clk); break;
    case 1: hipLaunchKernelGGL(bf16_probe<false>, grid, block, 0, st, iters, out, clk); break;
    case 2: hipLaunchKernelGGL(f32_probe<true>, grid, block, 0, st, iters, out, clk); break;
    case 3: hipLaunchKernelGGL(f32_probe<false>, grid, block, 0, st, iters, out, clk); break;
    case 4: hipLaunchKernelGGL(f64_probe<true>, grid, block, 0, st, iters, out, clk); break;
    case 5: hipLaunchKernelGGL(f64_probe<false>, grid, block, 0, st, iters, out, clk); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Copies `bytes` (a multiple of 16 KiB, both pointers 16-byte aligned) from src to dst on `stream`.
int kqp_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes <= 0 || bytes % 16384 != 0 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(dst) % 16)
    return -1;
  hipLaunchKernelGGL(copy_probe, dim3(256 * 16), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
