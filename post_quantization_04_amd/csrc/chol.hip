// Upper-triangular R with R^T R = (H + damp * mean(diag H) * I)^-1.
//
// With J the index-reversal permutation, J H~ J = L L^T (lower Cholesky) gives
// H~ = V V^T with V = J L J upper, and R = V^-1 = J L^-1 J. So the kernel
// chain is:
//   1. damping: delta = damp * mean(diag H) in float64;
//   2. reversal copy A = J H J + delta I into scratch, padded to a multiple of
//      64 with an identity block; M (which becomes L^-1) starts at zero;
//   3. blocked right-looking Cholesky of A with 64 x 64 blocks, and one step
//      behind it M = L^-1 by blocked forward substitution, in two levels:
//      super-panels of kSP = 4 blocks (256 columns). One launch per step
//      kb = 0 .. nb (the last one only finishes M):
//      * the diagonal role brings block column kb up to date with the
//        previous panel (float64 MFMA) when that panel belongs to the same
//        super-panel, factors and inverts the diagonal block in float64 in LDS
//        (every workgroup of the role does this itself); workgroup 0 stores
//        M_kk = L_kk^-1 and each other one multiplies one 64-row block of the
//        panel by L_kk^-T;
//      * the row role forms row j = kb - 1 of M, one 64 x 64 block per
//        workgroup, from the stored M_jj:
//          M[j, c] = -M_jj (S[j, c] + L[j, j-1] M[j-1, c]),   c < j,
//        where S[i, c] = sum over i' < i - 1 of L[i, i'] M[i', c] has been
//        accumulated in M's lower blocks by the earlier launches;
//      * the update role applies the previous panel (rank 64) only inside the
//        current super-panel: A[i, j'] -= L[i, kb-1] L[j', kb-1]^T for block
//        columns kb + 1 .. to the super-panel's end (every row below), and
//        S[i, c] += L[i, kb-2] M[kb-2, c] for the super-panel's rows from kb;
//      after the last step of a super-panel [s0, s1) one more launch applies
//      the whole super-panel at once (rank 256) to everything beyond it:
//        A[i, j] -= L[i, s0:s1] L[j, s0:s1]^T            for s1 <= j <= i,
//        S[i, c] += L[i, s0-1:s1-1] M[s0-1:s1-1, c]       for i >= s1
//      (the substitution runs one block behind the factor, so its panel is the
//      super-panel shifted by one block). Each element of the trailing matrix
//      is read and written once per super-panel instead of once per block, a
//      quarter of the HBM traffic of the one-level form. Products are 128 x 128
//      tiles: float32 MFMA (v_mfma_f32_32x32x2f32) inside a super-panel, and
//      for the rank-256 launches bfloat16 MFMA on an exact three-piece split of
//      each float32 operand (float32-level products at 2.7x the float32 rate);
//   4. R = J M J written over H (strict lower triangle zeroed).
// A pivot that is not positive and finite stops the chain: `info` takes the
// original index + 1 and every later kernel returns at once.
#include <type_traits>

#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kB = 64;  // block edge
constexpr int kSP = 4;  // blocks per super-panel

typedef float f32x16 __attribute__((ext_vector_type(16)));

// --------------------------------------------------------------------------
// 128 x 128 float32 MFMA tile product: C = alpha * A B + beta * C over k in [k0, k1)
//   A element (i, k) at a[i * lda + k]
//   B element (k, j) at b[k * ldb + j] (TB: b[j * ldb + k])
// k0 and k1 are multiples of 16, pointers and pitches 16-byte aligned;
// m_valid and n_valid are multiples of 64 (rows i >= m_valid of A and
// columns j >= n_valid of B read as zero and are not stored), so every
// validity test is uniform across a wave. 256 threads: 4 waves in a 2 x 2
// grid of 64 x 64, each a 2 x 2 grid of v_mfma_f32_32x32x2f32 blocks. k
// advances in chunks of 16 through two LDS buffers held k-major ([k][i],
// padded rows); the next chunk is loaded into registers while the current one
// is multiplied.
// --------------------------------------------------------------------------
constexpr int kG = 128;       // tile edge
constexpr int kGK = 16;       // k chunk
constexpr int kGP = kG + 4;   // LDS row pitch (floats)

struct GemmLds {
  float a[2][kGK][kGP];
  float b[2][kGK][kGP];
};

// Thread's share of a 128 x 16 chunk with rows along the contiguous axis of
// memory transposed into LDS: rows t / 4 and t / 4 + 64, k quad t % 4.
__device__ __forceinline__ void load_rows(const float* p, int64_t ld, int valid, int kc, float4 (&v)[2]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = (t >> 2) + 64 * h;
    v[h] = (64 * h < valid) ? *reinterpret_cast<const float4*>(p + int64_t(i) * ld + kc + 4 * (t & 3))
                            : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}
__device__ __forceinline__ void store_rows(float (*lds)[kGP], const float4 (&v)[2]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = (t >> 2) + 64 * h, k = 4 * (t & 3);
    lds[k][i] = v[h].x;
    lds[k + 1][i] = v[h].y;
    lds[k + 2][i] = v[h].z;
    lds[k + 3][i] = v[h].w;
  }
}
// 16 x 128 chunk with columns along the contiguous axis: k rows t / 32 and
// t / 32 + 8, column quad t % 32.
__device__ __forceinline__ void load_cols(const float* p, int64_t ld, int valid, int kc, float4 (&v)[2]) {
  const int t = threadIdx.x;
  const int j = 4 * (t & 31);  // a wave covers 64 columns of one k row pair
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = (t >> 5) + 8 * h;
    v[h] = ((j & ~63) < valid) ? *reinterpret_cast<const float4*>(p + int64_t(kc + k) * ld + j)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}
__device__ __forceinline__ void store_cols(float (*lds)[kGP], const float4 (&v)[2]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) *reinterpret_cast<float4*>(&lds[(t >> 5) + 8 * h][4 * (t & 31)]) = v[h];
}

template <bool TB>
__device__ __forceinline__ void gemm128(GemmLds& sm, const float* a, int64_t lda, const float* b, int64_t ldb, float* c, int64_t ldc,
                        int m_valid, int n_valid, int k0, int k1, float alpha, float beta) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
  // D of a 32 x 32 block: lane l, register r -> row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
  // Blocks are wholly valid or not. With beta != 0 the C block is read before the k loop, so
  // its latency hides behind the products.
  const bool rows_ok[2] = {wi * 64 < m_valid, wi * 64 + 32 < m_valid};
  const bool cols_ok[2] = {wj * 64 < n_valid, wj * 64 + 32 < n_valid};
  float* cp[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
      cp[x][y] = c + int64_t(wi * 64 + x * 32 + 4 * (lane >> 5)) * ldc + wj * 64 + y * 32 + (lane & 31);
  f32x16 old[2][2];
  if (beta != 0.0f) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        if (rows_ok[x] && cols_ok[y]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) old[x][y][r] = cp[x][y][int64_t(8 * (r >> 2) + (r & 3)) * ldc];
        }
  }
  const int nchunk = (k1 - k0) / kGK;
  float4 va[2], vb[2];
  auto load = [&](int kc) {
    load_rows(a, lda, m_valid, kc, va);
    if (TB) load_rows(b, ldb, n_valid, kc, vb);
    else load_cols(b, ldb, n_valid, kc, vb);
  };
  auto store = [&](int buf) {
    store_rows(sm.a[buf], va);
    if (TB) store_rows(sm.b[buf], vb);
    else store_cols(sm.b[buf], vb);
  };
  if (nchunk > 0) {
    load(k0);
    store(0);
  }
  __syncthreads();
  for (int ch = 0; ch < nchunk; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nchunk) load(k0 + (ch + 1) * kGK);
#pragma unroll
    for (int kk = 0; kk < kGK / 2; ++kk) {
      const int kr = 2 * kk + (lane >> 5);
      float fa[2], fb[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) fa[x] = sm.a[buf][kr][wi * 64 + x * 32 + (lane & 31)];
#pragma unroll
      for (int y = 0; y < 2; ++y) fb[y] = sm.b[buf][kr][wj * 64 + y * 32 + (lane & 31)];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    if (ch + 1 < nchunk) store(buf ^ 1);
    __syncthreads();
  }
  if (beta != 0.0f) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        if (rows_ok[x] && cols_ok[y]) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cp[x][y][int64_t(8 * (r >> 2) + (r & 3)) * ldc] = alpha * acc[x][y][r] + beta * old[x][y][r];
        }
  } else {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        if (rows_ok[x] && cols_ok[y]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) cp[x][y][int64_t(8 * (r >> 2) + (r & 3)) * ldc] = alpha * acc[x][y][r];
        }
  }
}

// ---------------------------------------------------------------------------
// The same 128 x 128 tile product with float32 operands on bfloat16 MFMA
// (v_mfma_f32_32x32x16_bf16, 16x the float32 MFMA rate): each operand x is
// split exactly into three round-to-nearest bfloat16 pieces, x = hi + mid + lo
// (8 + 8 + 8 significant bits), and the product takes the six piece products
// whose weight is at least 2^-16 of hi * hi: hi*hi, hi*mid, mid*hi, hi*lo,
// mid*mid, lo*hi. Each piece product is exact in float32 and accumulates in
// the MFMA's float32 accumulator, so the result carries float32-level
// rounding (the dropped terms are below 2^-24 relative). Staging as in gemm128
// (float32 chunks of 16 k, k-major in LDS); a lane's operand of one k-step is
// 8 consecutive k of one row (lanes 0-31: k 0..7, lanes 32-63: k 8..15).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Split3 {
  bf16x8 hi, mid, lo;
};

__device__ __forceinline__ Split3 split3(const float (&v)[8]) {
  Split3 s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(v[e]);
    const float r1 = v[e] - static_cast<float>(h);   // exact: below half a bfloat16 ulp of v
    const __bf16 m = static_cast<__bf16>(r1);
    const float r2 = r1 - static_cast<float>(m);     // exact, at most 8 significant bits
    s.hi[e] = h;
    s.mid[e] = m;
    s.lo[e] = static_cast<__bf16>(r2);               // exact
  }
  return s;
}

__device__ __forceinline__ f32x16 mfma_split(const Split3& a, const Split3& b, f32x16 acc) {
  // smallest terms first
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.lo, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.mid, b.mid, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b.lo, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.mid, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b.mid, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b.hi, acc, 0, 0, 0);
  return acc;
}

// The LDS of the split product: per buffer and operand the hi, mid and lo bfloat16 pieces of a
// 128 x 16 chunk as [row][k] tiles (pitch 24: eight consecutive rows on distinct banks for the
// 16-byte reads), each value split once when stored.
constexpr int kSplitPitch = kGK + 8;
struct SplitLds {
  alignas(16) __bf16 a[2][3][kG][kSplitPitch];
  alignas(16) __bf16 b[2][3][kG][kSplitPitch];
};

template <bool TB>
__device__ __forceinline__ void gemm128_split(SplitLds& sm, const float* a, int64_t lda, const float* b, int64_t ldb,
                                              float* c, int64_t ldc, int m_valid, int n_valid, int k0, int k1,
                                              float alpha, float beta) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
  const bool rows_ok[2] = {wi * 64 < m_valid, wi * 64 + 32 < m_valid};
  const bool cols_ok[2] = {wj * 64 < n_valid, wj * 64 + 32 < n_valid};
  float* cp[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
      cp[x][y] = c + int64_t(wi * 64 + x * 32 + 4 * (lane >> 5)) * ldc + wj * 64 + y * 32 + (lane & 31);
  f32x16 old[2][2];
  if (beta != 0.0f) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        if (rows_ok[x] && cols_ok[y]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) old[x][y][r] = cp[x][y][int64_t(8 * (r >> 2) + (r & 3)) * ldc];
        }
  }
  const int nchunk = (k1 - k0) / kGK;
  // A and (TB) B: thread t takes row t / 2 of the tile and 8 consecutive k from 8 (t % 2), two
  // 16-byte loads; B without TB: column t % 128 and the 8 k rows from 8 (t / 128), 8 loads along
  // the row. Rows (columns) past the valid count read row (column) 0 and are stored as zero.
  const int t = threadIdx.x;
  const int ar = t >> 1, ak = 8 * (t & 1);
  const int bj = t & 127, bk = 8 * (t >> 7);
  const bool a_in = ar < m_valid, b_in = TB ? ar < n_valid : bj < n_valid;
  const float* arow = a + int64_t(a_in ? ar : 0) * lda + ak;
  const float* brow = TB ? b + int64_t(b_in ? ar : 0) * ldb + ak : b + (b_in ? bj : 0);
  // two register sets: chunk c is loaded into set c % 2 two chunks ahead of its multiply, so its
  // loads stay in flight across a whole chunk of MFMAs (a single set left each chunk's load
  // latency exposed behind only the 24 MFMAs of the chunk before it)
  float va[2][8], vb[2][8];
  auto load = [&](auto set_c, int kc) {
    constexpr int S = decltype(set_c)::value;
    const float4 x0 = *reinterpret_cast<const float4*>(arow + kc);
    const float4 x1 = *reinterpret_cast<const float4*>(arow + kc + 4);
    va[S][0] = x0.x; va[S][1] = x0.y; va[S][2] = x0.z; va[S][3] = x0.w;
    va[S][4] = x1.x; va[S][5] = x1.y; va[S][6] = x1.z; va[S][7] = x1.w;
    if (TB) {
      const float4 y0 = *reinterpret_cast<const float4*>(brow + kc);
      const float4 y1 = *reinterpret_cast<const float4*>(brow + kc + 4);
      vb[S][0] = y0.x; vb[S][1] = y0.y; vb[S][2] = y0.z; vb[S][3] = y0.w;
      vb[S][4] = y1.x; vb[S][5] = y1.y; vb[S][6] = y1.z; vb[S][7] = y1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) vb[S][e] = brow[int64_t(kc + bk + e) * ldb];
    }
  };
  // each value split once, into the hi / mid / lo tiles the MFMAs read; set S goes to buffer S
  auto store = [&](auto set_c) {
    constexpr int S = decltype(set_c)::value;
    float x[8], y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = a_in ? va[S][e] : 0.0f;
      y[e] = b_in ? vb[S][e] : 0.0f;
    }
    const Split3 sa = split3(x), sb = split3(y);
    *reinterpret_cast<bf16x8*>(&sm.a[S][0][ar][ak]) = sa.hi;
    *reinterpret_cast<bf16x8*>(&sm.a[S][1][ar][ak]) = sa.mid;
    *reinterpret_cast<bf16x8*>(&sm.a[S][2][ar][ak]) = sa.lo;
    const int br = TB ? ar : bj, bc = TB ? ak : bk;
    *reinterpret_cast<bf16x8*>(&sm.b[S][0][br][bc]) = sb.hi;
    *reinterpret_cast<bf16x8*>(&sm.b[S][1][br][bc]) = sb.mid;
    *reinterpret_cast<bf16x8*>(&sm.b[S][2][br][bc]) = sb.lo;
  };
  // waits for this wave's LDS accesses only (a full __syncthreads would also wait for the
  // chunk loads still in flight)
  auto lds_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  // Every chunk issues the same loads (past the last chunk they re-read it and are not used), so
  // the wait before a split covers only the set it splits: a load under a condition would leave
  // the compiler a path where that set's loads are the newest, and it would wait for all loads.
  auto kc_of = [&](int c) { return k0 + (c < nchunk ? c : nchunk - 1) * kGK; };
  const int kb = 8 * (lane >> 5), ln = lane & 31;
  // chunk c: buffer and register set c % 2; its multiply, then chunk c + 1 into the other buffer
  auto chunk = [&](auto set_c, int c) {
    constexpr int S = decltype(set_c)::value;
    using Other = std::integral_constant<int, 1 - S>;
    load(set_c, kc_of(c + 2));  // set S went to LDS before chunk c
    Split3 fa[2], fb[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = wi * 64 + x * 32 + ln;
      fa[x].hi = *reinterpret_cast<const bf16x8*>(&sm.a[S][0][r][kb]);
      fa[x].mid = *reinterpret_cast<const bf16x8*>(&sm.a[S][1][r][kb]);
      fa[x].lo = *reinterpret_cast<const bf16x8*>(&sm.a[S][2][r][kb]);
    }
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int r = wj * 64 + y * 32 + ln;
      fb[y].hi = *reinterpret_cast<const bf16x8*>(&sm.b[S][0][r][kb]);
      fb[y].mid = *reinterpret_cast<const bf16x8*>(&sm.b[S][1][r][kb]);
      fb[y].lo = *reinterpret_cast<const bf16x8*>(&sm.b[S][2][r][kb]);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = mfma_split(fa[x], fb[y], acc[x][y]);
    // buffer 1 - S held chunk c - 1, whose reads finished before the last barrier
    if (c + 1 < nchunk) store(Other{});
    lds_sync();
  };
  if (nchunk > 0) {
    load(C0{}, kc_of(0));
    load(C1{}, kc_of(1));
    store(C0{});
    lds_sync();
    int ch = 0;
    for (; ch + 2 <= nchunk; ch += 2) {
      chunk(C0{}, ch);
      chunk(C1{}, ch + 1);
    }
    if (ch < nchunk) chunk(C0{}, ch);
  }
  if (beta != 0.0f) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        if (rows_ok[x] && cols_ok[y]) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cp[x][y][int64_t(8 * (r >> 2) + (r & 3)) * ldc] = alpha * acc[x][y][r] + beta * old[x][y][r];
        }
  } else {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        if (rows_ok[x] && cols_ok[y]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) cp[x][y][int64_t(8 * (r >> 2) + (r & 3)) * ldc] = alpha * acc[x][y][r];
        }
  }
}

__device__ __forceinline__ void tri(int t, int& I, int& J) {
  int i = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  I = i;
  J = t - i * (i + 1) / 2;
}

__global__ __launch_bounds__(256) void damp_kernel(const float* __restrict__ h, int64_t d, float damp,
                                                   double* __restrict__ delta, int32_t* __restrict__ info) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256) s += static_cast<double>(h[i * d + i]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *delta = static_cast<double>(damp) * red[0] / static_cast<double>(d);
    *info = 0;
  }
}

// A[i][j] = H[d-1-i][d-1-j] + delta [i == j]; identity outside d. M starts at
// 0: its lower blocks hold the running sums S of the substitution, and the
// blocks above its diagonal stay 0 (the far substitution update reads them).
__global__ void reverse_kernel(const float* __restrict__ h, int64_t d, int64_t dp, const double* __restrict__ delta,
                               float* __restrict__ a, float* __restrict__ m) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t i = blockIdx.y;
  if (j >= dp) return;
  float v;
  if (i < d && j < d) {
    v = h[(d - 1 - i) * d + (d - 1 - j)];
    if (i == j) v = static_cast<float>(static_cast<double>(v) + *delta);
  } else {
    v = (i == j) ? 1.0f : 0.0f;
  }
  a[i * dp + j] = v;
  m[i * dp + j] = 0.0f;
}

// ---------------------------------------------------------------------------
// Diagonal block factorization in float64 with 16 x 16 sub-blocks.
//   * base cases (16 x 16 Cholesky and its inverse) run on one wave, lanes
//     0..15 owning one row each in registers, columns broadcast through LDS;
//   * sub-panel, trailing and inverse products are float64 MFMA 16 x 16 x 4
//     (operands A[i][k] at lane i + 16 k, B[k][j] at lane j + 16 k; result
//     row 4 q + lane / 16, column lane % 16 in register q).
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kP = kB + 1;  // LDS row pitch (doubles)

// acc += A16 * B16 (or A16 * B16^T) for 16 x 16 tiles in LDS with pitch kP; one wave.
template <bool BT>
__device__ __forceinline__ f64x4 mm16(const double* a, const double* b, f64x4 acc) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const double fa = a[r * kP + 4 * kk + c];
    const double fb = BT ? b[r * kP + 4 * kk + c] : b[(4 * kk + c) * kP + r];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(fa, fb, acc, 0, 0, 0);
  }
  return acc;
}

// acc += A16 * B16^T with A16 float32 in LDS (pitch kP floats), B16 float64 (pitch kP).
__device__ __forceinline__ f64x4 mm16f(const float* a, const double* b, f64x4 acc) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(a[r * kP + 4 * kk + c]), b[r * kP + 4 * kk + c],
                                               acc, 0, 0, 0);
  return acc;
}

// acc += A16 * B16 with A16 float64 (pitch kP) and B16 float32 in LDS (pitch kP floats, [k][j]).
__device__ __forceinline__ f64x4 mm16df(const double* a, const float* b, f64x4 acc) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[r * kP + 4 * kk + c], static_cast<double>(b[(4 * kk + c) * kP + r]),
                                               acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ void store16(double* c, f64x4 v, double scale) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) c[(4 * q + (lane >> 4)) * kP + (lane & 15)] = scale * v[q];
}

__device__ __forceinline__ f64x4 load16(const double* c) {
  const int lane = threadIdx.x & 63;
  f64x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = c[(4 * q + (lane >> 4)) * kP + (lane & 15)];
  return v;
}

// Value of v in lane `src` of this lane's row of 16 (DPP row_newbcast; src a compile-time lane).
template <int CTRL>
__device__ __forceinline__ double dpp_row(double v) {
  // every lane reads a valid source under row_newbcast, so no "old" value is needed
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double bcast_row(double v, int src) {
  switch (src) {
    case 0: return dpp_row<0x150>(v);
    case 1: return dpp_row<0x151>(v);
    case 2: return dpp_row<0x152>(v);
    case 3: return dpp_row<0x153>(v);
    case 4: return dpp_row<0x154>(v);
    case 5: return dpp_row<0x155>(v);
    case 6: return dpp_row<0x156>(v);
    case 7: return dpp_row<0x157>(v);
    case 8: return dpp_row<0x158>(v);
    case 9: return dpp_row<0x159>(v);
    case 10: return dpp_row<0x15A>(v);
    case 11: return dpp_row<0x15B>(v);
    case 12: return dpp_row<0x15C>(v);
    case 13: return dpp_row<0x15D>(v);
    case 14: return dpp_row<0x15E>(v);
    default: return dpp_row<0x15F>(v);
  }
}

// 1 / sqrt(p) for finite p > 0: the hardware estimate refined by two Newton
// steps y <- y + y (1 - p y^2) / 2, which brings it to float64 rounding.
__device__ __forceinline__ double rsqrt_f64(double p) {
  double y = __builtin_amdgcn_rsq(p);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = fma(-p * y, y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return y;
}

// 16 x 16 Cholesky (lower) of the sub-block at l + o * (kP + 1) and its inverse
// into x + o * (kP + 1); wave 0 only. Each of the wave's four rows of 16
// lanes factors the block (lane i of a row holds row i in registers; columns
// are broadcast across the 16 lanes with DPP row_newbcast; pivots use
// 1 / sqrt(p), so the column chain has no division, square root, scalar round
// trip or LDS access); row q then forms the columns j = q mod 4 of the inverse.
// Returns the local index of the first bad pivot, or -1 (the chain runs to the
// end either way; a bad pivot only poisons values the caller then discards).
__device__ int base16(double* l, double* x, int o) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, q = lane >> 4;
  double* L = l + o * (kP + 1);
  double* X = x + o * (kP + 1);
  double r[16], y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) r[j] = L[i * kP + j];
  // Factor: after step k, lanes i >= k hold l_ik in r[k]. Lanes i < j also
  // update their (upper) r[j]; those values are never broadcast and are
  // cleared when their column comes up.
  int bad = -1;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const double p = bcast_row(r[k], k);
    bad = (bad < 0 && !(p > 0.0 && p < __builtin_huge_val())) ? k : bad;
    y[k] = rsqrt_f64(p);
    const double lik = (i == k) ? p * y[k] : r[k] * y[k];
    r[k] = (i >= k) ? lik : 0.0;
#pragma unroll
    for (int j = k + 1; j < 16; ++j) r[j] = fma(-lik, bcast_row(lik, j), r[j]);
  }
  bad = __builtin_amdgcn_readfirstlane(bad);
  if (bad >= 0) return bad;
  // Inverse by forward substitution, columns j = 4 c + q of X = L^-1 in row q:
  // xr[c] = X[i][4 c + q]. At step k row k of X is scaled by 1 / l_kk = y_k,
  // then removed from the rows below (columns beyond k are still zero).
  double xr[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) xr[c] = (i == 4 * c + q) ? 1.0 : 0.0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    constexpr int kc = 4;
    const int nc = (k >> 2) + 1 < kc ? (k >> 2) + 1 : kc;  // columns 4 c + q <= k need c <= k / 4
#pragma unroll
    for (int c = 0; c < nc; ++c) xr[c] = (i == k) ? xr[c] * y[k] : xr[c];
    const double lik = (i > k) ? r[k] : 0.0;
#pragma unroll
    for (int c = 0; c < nc; ++c) xr[c] = fma(-lik, bcast_row(xr[c], k), xr[c]);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = 4 * c + q;
    L[i * kP + j] = (j <= i) ? r[j] : 0.0;
    X[i * kP + j] = (j <= i) ? xr[c] : 0.0;
  }
  return -1;
}

// Shared memory of the diagonal role: the diagonal block, its inverse, the
// previous panel's rows of this block, and this workgroup's operand block with
// its second operand (float32): a panel block and its previous-panel rows, or
// a block S[kb, c] and the block M[kb-1, c].
struct DiagLds {
  double l[kB * kP];
  double x[kB * kP];
  double lp[kB * kP];
  double pb[kB * kP];
  float lb[kB * kP];
  int bad;
};

union StepLds {
  DiagLds dg;
  GemmLds gm;
};

// Diagonal role of step kb, workgroup b in [0, 1 + rest): brings block
// column kb up to date with the previous step's rank-64 update (L[:, kb-1],
// in float64 MFMA), factors the diagonal block and inverts its factor (every
// workgroup does this itself), then workgroup 0 writes L_kk^-1 to M, and
// workgroup b >= 1 writes L[kb + b, kb] = A[kb + b, kb] L_kk^-T. No workgroup
// writes a block another one of the launch reads, so the result does not
// depend on when each workgroup starts. All global reads are issued up front;
// the panel block's own update runs on waves 1..3 while wave 0 factors the
// first 16 columns.
__device__ void diag_role(DiagLds& sm, float* __restrict__ a, float* __restrict__ m, int64_t dp, int kb, int64_t d,
                          int32_t* __restrict__ info, int b) {
  double* l = sm.l;
  double* x = sm.x;
  double* lp = sm.lp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t o = int64_t(kb) * kB, op = o - kB;
  const int64_t r0 = o + int64_t(b) * kB;
  // the previous panel's update is deferred to here only inside a super-panel; at a super-panel's
  // first block the far launch before this one has applied it
  const bool panel = b > 0, prev = (kb % kSP) != 0;
  // this thread's 16 elements e = tid + 256 q of the diagonal block, its previous-panel
  // rows, the panel block and its previous-panel rows: every load is issued before the
  // first LDS write, so the inputs written by the previous launch arrive in one round trip
  float dg[16], dq[16], ab[16], lb[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    dg[q] = a[(o + (e >> 6)) * dp + o + (e & 63)];
    dq[q] = prev ? a[(o + (e >> 6)) * dp + op + (e & 63)] : 0.0f;
  }
  if (panel) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q;
      ab[q] = a[(r0 + (e >> 6)) * dp + o + (e & 63)];
      lb[q] = prev ? a[(r0 + (e >> 6)) * dp + op + (e & 63)] : 0.0f;
    }
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q, i = e >> 6, j = e & 63;
    l[i * kP + j] = j <= i ? static_cast<double>(dg[q]) : 0.0;
    x[i * kP + j] = 0.0;
    if (prev) lp[i * kP + j] = static_cast<double>(dq[q]);
  }
  if (panel) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q;
      sm.pb[(e >> 6) * kP + (e & 63)] = static_cast<double>(ab[q]);
      sm.lb[(e >> 6) * kP + (e & 63)] = lb[q];
    }
  }
  if (tid == 0) sm.bad = -1;
  __syncthreads();
  if (prev) {
    // A_kk -= L[kb, kb-1] L[kb, kb-1]^T on the 10 lower 16 x 16 tiles
    for (int q = wave; q < 10; q += 4) {
      int tt = 0, uu = 0, n = 0;
      for (int ti = 0; ti < 4; ++ti)
        for (int ui = 0; ui <= ti; ++ui, ++n)
          if (n == q) { tt = ti; uu = ui; }
      f64x4 acc = f64x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mm16<true>(lp + 16 * tt * kP + 16 * ks, lp + 16 * uu * kP + 16 * ks, acc);
      const f64x4 c = load16(l + 16 * tt * kP + 16 * uu);
      store16(l + 16 * tt * kP + 16 * uu, c - acc, 1.0);
    }
    __syncthreads();
  }
  for (int s = 0; s < 4; ++s) {
    if (wave == 0) {
      const int bb = base16(l, x, 16 * s);
      if (lane == 0 && bb >= 0) sm.bad = 16 * s + bb;
    } else if (s == 0 && panel && prev) {
      // panel block -= L[r0.., kb-1] L[kb, kb-1]^T (16 tiles over waves 1..3)
      for (int q = wave - 1; q < 16; q += 3) {
        const int ti = q >> 2, tj = q & 3;
        f64x4 acc = f64x4{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mm16f(sm.lb + 16 * ti * kP + 16 * ks, lp + 16 * tj * kP + 16 * ks, acc);
        store16(sm.pb + 16 * ti * kP + 16 * tj, load16(sm.pb + 16 * ti * kP + 16 * tj) - acc, 1.0);
      }
    }
    __syncthreads();
    if (sm.bad >= 0) {
      if (tid == 0 && b == 0) {
        const int64_t ir = o + sm.bad;
        atomicCAS(info, 0, static_cast<int32_t>(((ir < d) ? d - 1 - ir : ir) + 1));
      }
      return;
    }
    // sub-panel: L[t][s] = A[t][s] inv(L_ss)^T for t > s (one tile per wave)
    const int t = s + 1 + wave;
    f64x4 v = f64x4{};
    if (t < 4) v = mm16<true>(l + 16 * t * kP + 16 * s, x + 16 * s * kP + 16 * s, v);
    __syncthreads();
    if (t < 4) store16(l + 16 * t * kP + 16 * s, v, 1.0);
    __syncthreads();
    // trailing: A[t][u] -= L[t][s] L[u][s]^T for s < u <= t (at most 6 tiles)
    for (int q = wave; q < 6; q += 4) {
      int tt = 0, uu = 0, n = 0;
      for (int ti = s + 1; ti < 4; ++ti)
        for (int ui = s + 1; ui <= ti; ++ui, ++n)
          if (n == q) { tt = ti; uu = ui; }
      if (q < n) {
        f64x4 c = load16(l + 16 * tt * kP + 16 * uu);
        f64x4 pp = mm16<true>(l + 16 * tt * kP + 16 * s, l + 16 * uu * kP + 16 * s, f64x4{});
        store16(l + 16 * tt * kP + 16 * uu, c - pp, 1.0);
      }
    }
    __syncthreads();
  }
  // inverse: M[t][s] = -inv(L_tt) sum_{u = s}^{t - 1} L[t][u] M[u][s], row block by row block
  for (int t = 1; t < 4; ++t) {
    const int s = wave;  // one column block per wave
    f64x4 acc = f64x4{};
    if (s < t) {
      for (int u = s; u < t; ++u) acc = mm16<false>(l + 16 * t * kP + 16 * u, x + 16 * u * kP + 16 * s, acc);
    }
    __syncthreads();
    if (s < t) store16(x + 16 * t * kP + 16 * s, acc, 1.0);  // temporary: T = sum L M
    __syncthreads();
    f64x4 mv = f64x4{};
    if (s < t) mv = mm16<false>(x + 16 * t * kP + 16 * t, x + 16 * t * kP + 16 * s, f64x4{});
    __syncthreads();
    if (s < t) store16(x + 16 * t * kP + 16 * s, mv, -1.0);
    __syncthreads();
  }
  if (b == 0) {
    // L_kk^-1 into M. L_kk itself stays out of A: no later kernel reads a
    // diagonal block of L, and every workgroup of this launch reads A_kk from
    // A, possibly after this one has finished.
    for (int e = tid; e < kB * kB; e += 256) {
      const int i = e >> 6, j = e & 63;
      m[(o + i) * dp + o + j] = static_cast<float>(x[i * kP + j]);
    }
    return;
  }
  // P = A[r0.., kb] L_kk^-T, 64 x 64 x 64 in float64 MFMA (4 x 4 tiles of 16, wave w owns tile row w)
  f64x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ti = wave, tj = q;
    f64x4 c = f64x4{};
    for (int u = 0; u <= tj; ++u)  // (L_kk^-T)[u][tj] = M[tj][u], zero for u > tj
      c = mm16<true>(sm.pb + 16 * ti * kP + 16 * u, x + 16 * tj * kP + 16 * u, c);
    acc[q] = c;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = 16 * wave + 4 * w + (lane >> 4), j = 16 * q + (lane & 15);
      a[(r0 + i) * dp + o + j] = static_cast<float>(acc[q][w]);
    }
  }
}

// Row role: block c < j of row j >= 1 of M = L^-1,
//   M[j, c] = -M_jj (S[j, c] + L[j, j-1] M[j-1, c]),
// in float64 MFMA from float32 operands; M_jj, L[j, j-1] and M[j-1, c] were
// stored by earlier launches, S[j, c] is complete (its last term is the one
// added here).
__device__ void row_role(DiagLds& sm, const float* __restrict__ a, float* __restrict__ m, int64_t dp, int j, int c) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t o = int64_t(j) * kB, op = o - kB, c0 = int64_t(c) * kB;
  float sv[16], lv[16], xv[16], mv[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q, i = e >> 6, jj = e & 63;
    sv[q] = m[(o + i) * dp + c0 + jj];   // S[j, c]
    lv[q] = a[(o + i) * dp + op + jj];   // L[j, j-1]
    xv[q] = m[(op + i) * dp + c0 + jj];  // M[j-1, c]
    mv[q] = m[(o + i) * dp + o + jj];    // M_jj
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q, i = e >> 6, jj = e & 63;
    sm.pb[i * kP + jj] = static_cast<double>(sv[q]);
    sm.lp[i * kP + jj] = static_cast<double>(lv[q]);
    sm.lb[i * kP + jj] = xv[q];
    sm.x[i * kP + jj] = static_cast<double>(mv[q]);
  }
  __syncthreads();
  // P = S + L[j, j-1] M[j-1, c]: wave w owns tile row w
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f64x4 acc = load16(sm.pb + 16 * wave * kP + 16 * q);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mm16df(sm.lp + 16 * wave * kP + 16 * ks, sm.lb + 16 * ks * kP + 16 * q, acc);
    store16(sm.l + 16 * wave * kP + 16 * q, acc, 1.0);
  }
  __syncthreads();
  // M[j, c] = -M_jj P (M_jj lower: tile row w needs tile rows u <= w of P)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f64x4 acc = f64x4{};
    for (int u = 0; u <= wave; ++u) acc = mm16<false>(sm.x + 16 * wave * kP + 16 * u, sm.l + 16 * u * kP + 16 * q, acc);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = 16 * wave + 4 * w + (lane >> 4), jj = 16 * q + (lane & 15);
      m[(o + i) * dp + c0 + jj] = static_cast<float>(-acc[w]);
    }
  }
}

// Update role of step kb, tile u, inside super-panel [s0, s1) (block indices).
// Tiles u < n_a (kb > s0): A[i, j] -= L[i, kb-1] L[j, kb-1]^T for block
// columns kb + 1 <= j < s1 and every row from kb + 1 on (a strip of at most 128
// columns; a tile that crosses the diagonal also rewrites part of A's upper
// triangle, which is never read); block column kb receives the same update in
// the diagonal role. Tiles u >= n_a (kb > s0, kb >= 2): S[i, c] += L[i, kb-2]
// M[kb-2, c] for row blocks kb <= i < s1 and column blocks c <= kb - 2; row kb -
// 1 takes this term in the row role, rows from s1 on in the far launch.
__device__ void update_role(GemmLds& sm, float* __restrict__ a, float* __restrict__ m, int64_t dp, int kb, int s1,
                            int u, int n_a) {
  if (u < n_a) {
    const int64_t c0 = int64_t(kb + 1) * kB;
    const int64_t ri = c0 + int64_t(u) * kG;
    const int mv = static_cast<int>(dp - ri < kG ? dp - ri : kG);
    const int nv = (s1 - kb - 1) * kB;  // 64 or 128
    const int64_t op = int64_t(kb - 1) * kB;
    gemm128<true>(sm, a + ri * dp + op, dp, a + c0 * dp + op, dp, a + ri * dp + c0, dp, mv, nv, 0, kB, -1.0f, 1.0f);
    return;
  }
  u -= n_a;
  const int ncol = kb / 2;  // 128-wide tiles over columns [0, 64 (kb - 1))
  const int64_t o2 = int64_t(kb - 2) * kB;
  const int64_t ri = int64_t(kb) * kB + int64_t(u / ncol) * kG, cj = int64_t(u % ncol) * kG;
  const int64_t rend = int64_t(s1) * kB, cend = int64_t(kb - 1) * kB;
  const int mv = static_cast<int>(rend - ri < kG ? rend - ri : kG);
  const int nv = static_cast<int>(cend - cj < kG ? cend - cj : kG);
  gemm128<false>(sm, a + ri * dp + o2, dp, m + o2 * dp + cj, dp, m + ri * dp + cj, dp, mv, nv, 0, kB, 1.0f, 1.0f);
}

// Step kb of the blocked factorization and substitution: workgroups
// [0, n_diag) take the diagonal role, the next n_row the row role (row kb - 1
// of M), the rest the update role. The roles write disjoint blocks (block
// column kb of A and diagonal block kb of M; row kb - 1 of M; the super-panel's
// columns beyond kb of A and its rows from kb on of M) and read none that
// another role of the launch writes, so one launch per step suffices.
__global__ __launch_bounds__(256) void chol_step_kernel(float* __restrict__ a, float* __restrict__ m, int64_t dp, int kb,
                                                        int64_t d, int s1, int n_diag, int n_row, int n_a,
                                                        int32_t* __restrict__ info) {
  __shared__ StepLds sm;
  if (*info) return;
  const int b = static_cast<int>(blockIdx.x);
  if (b < n_diag) diag_role(sm.dg, a, m, dp, kb, d, info, b);
  else if (b < n_diag + n_row) row_role(sm.dg, a, m, dp, kb - 1, b - n_diag);
  else update_role(sm.gm, a, m, dp, kb, s1, b - n_diag - n_row, n_a);
}

// Rank-256 update of everything beyond super-panel [s0, s1): tiles u < n_a
// take the lower triangle of A's trailing block (128 x 128 tiles from block
// s1 on), A[i, j] -= L[i, s0:s1] L[j, s0:s1]^T; the others take S[i, c] +=
// L[i, k0:k1] M[k0:k1, c] for rows from block s1 on and column blocks below
// s1 - 1, with k0 = max(s0 - 1, 0) and k1 = s1 - 1 (the substitution's panel,
// one block behind; M is zero above its diagonal blocks, so columns beyond a
// row's diagonal add nothing). The two roles write disjoint blocks and read
// none that the other writes.
// Tiles run in super-blocks of kFarSB x kFarSB tiles, dealt to the XCDs in turn (workgroups are
// dispatched to the XCDs round robin; two workgroups per CU give an XCD 64 at once, one
// super-block): the 64 tiles running together on an XCD read 8 + 8 panel strips (128 KB each)
// through its L2 instead of two each from beyond it. Super-blocks 0 .. n_sa - 1 cover the lower
// triangle of the trailing A (ntu tiles a side), the rest the ntu x ncol rectangle of M.
constexpr int kFarSB = 8;
constexpr int kFarXcds = 8;

__global__ __launch_bounds__(256) void chol_far_kernel(float* __restrict__ a, float* __restrict__ m, int64_t dp, int s0,
                                                       int s1, int ntu, int ncol, int n_sa, int n_sm,
                                                       int32_t* __restrict__ info) {
  __shared__ SplitLds sm;
  if (*info) return;
  const int xcd = static_cast<int>(blockIdx.x) % kFarXcds, local = static_cast<int>(blockIdx.x) / kFarXcds;
  const int sb = (local / (kFarSB * kFarSB)) * kFarXcds + xcd, within = local % (kFarSB * kFarSB);
  if (sb >= n_sa + n_sm) return;
  const int64_t r0 = int64_t(s1) * kB;
  if (sb < n_sa) {
    int P, Q;
    tri(sb, P, Q);
    const int I = P * kFarSB + within / kFarSB, J = Q * kFarSB + within % kFarSB;
    if (I >= ntu || J > I) return;
    const int64_t ri = r0 + int64_t(I) * kG, rj = r0 + int64_t(J) * kG;
    const int mv = static_cast<int>(dp - ri < kG ? dp - ri : kG);
    const int nv = static_cast<int>(dp - rj < kG ? dp - rj : kG);
    const int64_t k0 = int64_t(s0) * kB;
    gemm128_split<true>(sm, a + ri * dp + k0, dp, a + rj * dp + k0, dp, a + ri * dp + rj, dp, mv, nv, 0,
                  (s1 - s0) * kB, -1.0f, 1.0f);
    return;
  }
  const int v = sb - n_sa;
  const int ncsb = (ncol + kFarSB - 1) / kFarSB;
  const int I = (v / ncsb) * kFarSB + within / kFarSB, J = (v % ncsb) * kFarSB + within % kFarSB;
  if (I >= ntu || J >= ncol) return;
  const int64_t cend = int64_t(s1 - 1) * kB;
  const int64_t ri = r0 + int64_t(I) * kG, cj = int64_t(J) * kG;
  const int mv = static_cast<int>(dp - ri < kG ? dp - ri : kG);
  const int nv = static_cast<int>(cend - cj < kG ? cend - cj : kG);
  const int kb0 = s0 > 0 ? s0 - 1 : 0;
  const int64_t k0 = int64_t(kb0) * kB;
  gemm128_split<false>(sm, a + ri * dp + k0, dp, m + k0 * dp + cj, dp, m + ri * dp + cj, dp, mv, nv, 0,
                 (s1 - 1 - kb0) * kB, 1.0f, 1.0f);
}

// R[i][j] = M[d-1-i][d-1-j] for i <= j, 0 below the diagonal.
__global__ void output_kernel(const float* __restrict__ m, int64_t d, int64_t dp, float* __restrict__ h) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t i = blockIdx.y;
  if (j >= d) return;
  h[i * d + j] = (i <= j) ? m[(d - 1 - i) * dp + (d - 1 - j)] : 0.0f;
}

struct Layout {
  int64_t dp;
  size_t a_off, m_off, delta_off, total;
};

Layout layout(int64_t d) {
  Layout l{};
  l.dp = (d + kB - 1) / kB * kB;
  const size_t mat = align_up(size_t(l.dp) * l.dp * sizeof(float), 256);
  l.a_off = 0;
  l.m_off = mat;
  l.delta_off = 2 * mat;
  l.total = 2 * mat + 256;
  return l;
}

}  // namespace

size_t chol_workspace(int64_t d) { return layout(d).total; }

kq_status chol_run(float* h, int64_t d, float damp, int32_t* info, void* ws, hipStream_t st) {
  const Layout L = layout(d);
  char* base = static_cast<char*>(ws);
  float* a = reinterpret_cast<float*>(base + L.a_off);
  float* m = reinterpret_cast<float*>(base + L.m_off);
  double* delta = reinterpret_cast<double*>(base + L.delta_off);
  const int64_t dp = L.dp;
  const int nb = static_cast<int>(dp / kB);
  kq_status r;

  {
    LaunchTimer timer("damp_kernel", st);
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, st, h, d, damp, delta, info);
  }
  if ((r = check_launch("damp_kernel")) != KQ_OK) return r;
  // M is never read above its diagonal 64 x 64 blocks; its lower triangle is cleared here.
  {
    LaunchTimer timer("reverse_kernel", st);
    hipLaunchKernelGGL(reverse_kernel, dim3(static_cast<unsigned>((dp + 255) / 256), static_cast<unsigned>(dp)),
                       dim3(256), 0, st, h, d, dp, delta, a, m);
  }
  if ((r = check_launch("reverse_kernel")) != KQ_OK) return r;

  for (int kb = 0; kb <= nb; ++kb) {
    const int rest = nb - kb - 1;
    const int s0 = kb / kSP * kSP;
    const int s1 = s0 + kSP < nb ? s0 + kSP : nb;
    const bool inner = kb > s0 && kb < nb;  // the previous panel belongs to this super-panel
    const int n_diag = kb < nb ? 1 + rest : 0;
    const int n_row = kb >= 2 ? kb - 1 : 0;  // blocks c < j of row j = kb - 1 of M
    // strip of A: block columns kb + 1 .. s1 - 1 (at most 128 wide), 128-row tiles from block kb + 1
    const int n_a = (inner && kb + 1 < s1) ? static_cast<int>((dp - int64_t(kb + 1) * kB + kG - 1) / kG) : 0;
    // S rows kb .. s1 - 1 (128-row tiles) x 128-wide column tiles below 64 (kb - 1)
    const int n_s = (inner && kb >= 2) ? ((s1 - kb) * kB + kG - 1) / kG * (kb / 2) : 0;
    const int grid = n_diag + n_row + n_a + n_s;
    if (grid > 0) {
      {
        LaunchTimer timer("chol_step_kernel", st);
        hipLaunchKernelGGL(chol_step_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, a, m, dp, kb, d, s1,
                           n_diag, n_row, n_a, info);
      }
      if ((r = check_launch("chol_step_kernel")) != KQ_OK) return r;
    }
    if (kb + 1 == s1 && s1 < nb) {
      // the super-panel [s0, s1) is factored (and M one block behind it): apply it beyond s1
      const int64_t nrem = dp - int64_t(s1) * kB;
      const int ntu = static_cast<int>((nrem + kG - 1) / kG);
      const int ncol = static_cast<int>((int64_t(s1 - 1) * kB + kG - 1) / kG);
      const int nsb = (ntu + kFarSB - 1) / kFarSB;
      const int n_sa = nsb * (nsb + 1) / 2;
      const int n_sm = nsb * ((ncol + kFarSB - 1) / kFarSB);
      // every XCD runs the same number of super-block slots (the surplus workgroups return at once)
      const int64_t blocks = int64_t((n_sa + n_sm + kFarXcds - 1) / kFarXcds) * kFarXcds * kFarSB * kFarSB;
      {
        LaunchTimer timer("chol_far_kernel", st);
        hipLaunchKernelGGL(chol_far_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a, m, dp, s0, s1,
                           ntu, ncol, n_sa, n_sm, info);
      }
      if ((r = check_launch("chol_far_kernel")) != KQ_OK) return r;
    }
  }

  {
    LaunchTimer timer("output_kernel", st);
    hipLaunchKernelGGL(output_kernel, dim3(static_cast<unsigned>((d + 255) / 256), static_cast<unsigned>(d)),
                       dim3(256), 0, st, m, d, dp, h);
  }
  return check_launch("output_kernel");
}

}  // namespace kq
