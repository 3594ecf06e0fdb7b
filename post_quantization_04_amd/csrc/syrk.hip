// H = alpha * A^T A + beta * H for token-major bf16 A on gfx950 bf16 MFMA.
//
// A is [rows, d]: tokens by channels, channels contiguous. The contraction
// runs over tokens, so each MFMA operand needs consecutive tokens of one
// channel per lane. Panels of 32 tokens x 256 channels are copied straight
// from global memory into LDS in their natural token-major layout
// (global_load_lds_dwordx4, no register staging), and the MFMA fragments are
// read with the gfx950 transposing LDS load ds_read_b64_tr_b16: in each group
// of 16 lanes, four lanes per token supply 16 consecutive channels and lane j
// receives channel j at the four tokens. Two such loads give the eight tokens
// of a v_mfma_f32_32x32x16_bf16 operand. The 16-byte chunks of each 512-byte
// token row are XOR-swizzled with the token index so that both the DMA writes
// and the transposing reads run at the LDS bank minimum.
//
// Pipeline: four 32 KB stage buffers (both panels of 32 tokens; a diagonal
// tile loads its one panel twice) form a ring in LDS. Loads run three stages
// ahead (two stages in flight when a stage is awaited; a deeper ring measured
// no faster). Each buffer is its own __shared__ object and the ring is
// unrolled, so the compiler can tell the buffer being read from the ones
// being filled and does not drain the DMA queue before each LDS read. Before
// the one barrier per stage, each wave waits (vmcnt) only for its own loads
// of the next stage. Fragments are double buffered in registers: the reads of
// the next k-step are interleaved with the MFMAs of the current one, and the
// first reads of the next stage are issued right after the barrier, in the
// middle of the last k-step, together with the refill of the buffer just
// consumed.
//
// A final partial stage is loaded from the last 32 tokens of the slice and
// the rows already counted by the previous stage are zeroed in LDS; the stage
// count is padded to whole rings with zeroed stages (a full 8192-token slice
// is exactly 64 rings). Rows that are not 16-byte aligned, or fewer than 32
// rows in all, take a plain register-staged kernel.
//
// Work item = (lower-triangle 256 x 256 output tile, token slice of 8192
// rows). Each workgroup sums one slice in float32 MFMA accumulators (bf16
// products are exact) and writes the float32 partial tile. A second kernel
// adds the slices of a tile in float64, applies alpha and beta, rounds once to
// float32 and writes both triangles. Short float32 runs keep the accumulated
// rounding near 1e-7 relative, which the downstream column sweep needs.
//
// Workgroups are dispatched round robin over the 8 XCDs. With at least 8
// slices, XCD x runs every tile of slices x, x + 8, ..., tiles in a blocked
// order (4 tile rows x 8 tile columns, so the 32 workgroups of an XCD share
// about 12 channel panels) and each token slice streams through one L2 only.
// With fewer slices, the blocked tile list is cut into 8 groups and XCD x
// runs group x of every slice.
#include <utility>

#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kT = 256;          // output tile edge (channels)
constexpr int kKT = 32;          // tokens per LDS stage
constexpr int kNB = 4;           // stage buffers in the ring (2..8)
// tokens per float32 partial sum: whole rings, at most 8192 tokens
constexpr int kSlice = 8192 / (kNB * kKT) * (kNB * kKT);
constexpr int kThreads = 256;    // 4 waves in a 2 x 2 grid, 128 x 128 outputs each
constexpr int kPanelUnits = kT * kKT * 2 / 16;  // 16-byte units per LDS panel (1024)
constexpr int kPanelBytes = kPanelUnits * 16;
constexpr int kUnitsPerLane = kPanelUnits / kThreads;  // DMA loads per lane per panel (4)
constexpr int kTargetItems = 8192;  // work items per launch before slices are split into groups

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

#define KQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define KQ_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))

// The ring: one __shared__ object per stage buffer, panel I then panel J
// (only the first kNB are referenced, and only those are allocated).
[[maybe_unused]] __shared__ uint4 ring0[2 * kPanelUnits];
[[maybe_unused]] __shared__ uint4 ring1[2 * kPanelUnits];
[[maybe_unused]] __shared__ uint4 ring2[2 * kPanelUnits];
[[maybe_unused]] __shared__ uint4 ring3[2 * kPanelUnits];
[[maybe_unused]] __shared__ uint4 ring4[2 * kPanelUnits];
[[maybe_unused]] __shared__ uint4 ring5[2 * kPanelUnits];
[[maybe_unused]] __shared__ uint4 ring6[2 * kPanelUnits];
[[maybe_unused]] __shared__ uint4 ring7[2 * kPanelUnits];
static_assert(kNB >= 2 && kNB <= 8 && kNB * 2 * kPanelUnits * 16 <= 160 * 1024, "ring must fit in LDS");

template <int K>
__device__ __forceinline__ uint4* ring() {
  static_assert(K >= 0 && K < kNB, "ring index");
  if constexpr (K == 0) return ring0;
  else if constexpr (K == 1) return ring1;
  else if constexpr (K == 2) return ring2;
  else if constexpr (K == 3) return ring3;
  else if constexpr (K == 4) return ring4;
  else if constexpr (K == 5) return ring5;
  else if constexpr (K == 6) return ring6;
  else return ring7;
}

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

// Byte offset (inside a panel) of this lane's first transposing read for the
// operand block starting at channel ch0; k-step kk adds 8192 bytes, the second
// read of a pair (+4 tokens) adds 2048.
__device__ __forceinline__ int32_t tr_offset(int ch0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int ch = ch0 + 16 * (g & 1) + 4 * (j & 3);
  const int cc = ch >> 3, half = (ch >> 2) & 1;
  const int tb = 8 * (g >> 1) + (j >> 2);
  return slot(tb, cc) * 16 + half * 8;
}

__device__ __forceinline__ bf16x8 frag_at(const char* p) {
  const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)KQ_LDS(p));
  const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)KQ_LDS(p + 2048));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 r = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Operand fragments of one 16-token k-step: 4 row blocks of the wave's I
// range, 4 column blocks of its J range.
struct Frags {
  bf16x8 a[4], b[4];
};

__device__ __forceinline__ void read_frags(const char* buf, int kk, const int32_t (&oa)[4], const int32_t (&ob)[4],
                                           Frags& f) {
#pragma unroll
  for (int x = 0; x < 4; ++x) f.a[x] = frag_at(buf + oa[x] + kk * 8192);
#pragma unroll
  for (int y = 0; y < 4; ++y) f.b[y] = frag_at(buf + ob[y] + kk * 8192);
}

// MFMAs of row blocks x0 .. x1 - 1 against all 4 column blocks.
__device__ __forceinline__ void mfma_rows(const Frags& f, int x0, int x1, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int x = x0; x < x1; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
      acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[x], f.b[y], acc[x][y], 0, 0, 0);
}

// Per-lane byte offsets (from a stage origin a + t0 * lda) of the chunks this
// lane copies into a panel: load i of wave w fills slot w * 256 + i * 64 +
// lane, whose chunk is the un-swizzled position. Chunks past channel d re-read
// the row's last 8 channels (their outputs are discarded).
__device__ __forceinline__ void dma_offsets(int64_t lda, int64_t d, int64_t c0, uint32_t (&off)[kUnitsPerLane]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kUnitsPerLane; ++i) {
    const int sl = wave * (kUnitsPerLane * 64) + i * 64 + lane;
    const int t = sl >> 5, cs = sl & 31;
    const int cc = (cs & 16) | ((cs & 15) ^ ((t & 3) << 2));
    int64_t ch = c0 + int64_t(cc) * 8;
    if (ch > d - 8) ch = d - 8;
    off[i] = static_cast<uint32_t>((int64_t(t) * lda + ch) * 2);
  }
}

// Issues the DMA copies of one stage (both panels) into ring buffer K.
template <int K>
__device__ __forceinline__ void dma_stage(const char* origin, const uint32_t (&da)[kUnitsPerLane],
                                          const uint32_t (&db)[kUnitsPerLane], int wave) {
  uint4* dst = ring<K>() + wave * (kUnitsPerLane * 64);
#pragma unroll
  for (int i = 0; i < kUnitsPerLane; ++i)
    __builtin_amdgcn_global_load_lds(KQ_GLOBAL(origin + da[i]), KQ_LDS(dst + i * 64), 16, 0, 0);
#pragma unroll
  for (int i = 0; i < kUnitsPerLane; ++i)
    __builtin_amdgcn_global_load_lds(KQ_GLOBAL(origin + db[i]), KQ_LDS(dst + kPanelUnits + i * 64), 16, 0, 0);
}

// Workgroup barrier without the full memory drain of __syncthreads (which
// would also wait for the loads of the stages still in flight).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Uniform per-workgroup state of the ring kernel.
struct Ring {
  const char* a;        // A as bytes
  int64_t lda2;         // row pitch in bytes
  int64_t tok_begin, tok_end;
  int nstage;
  int wave;
  uint32_t da[kUnitsPerLane], db[kUnitsPerLane];
  int32_t oa[4], ob[4];

  // First token copied for stage q: a partial last stage is shifted back to
  // end at tok_end, and stages past the end (which pad the count to whole
  // rings and keep the number of copies in flight constant) repeat the last
  // stage and are zeroed once landed.
  __device__ __forceinline__ int64_t origin_token(int q) const {
    const int qq = q < nstage ? q : nstage - 1;
    const int64_t t0 = tok_begin + int64_t(qq) * kKT;
    return t0 + kKT <= tok_end ? t0 : tok_end - kKT;
  }
  template <int K>
  __device__ __forceinline__ void issue(int q) const {
    dma_stage<K>(a + origin_token(q) * lda2, da, db, wave);
  }
  // Makes stage q (in ring buffer K) visible to all waves, with the copies of
  // the kNB - 2 following stages still in flight. The rows of a partial stage
  // that precede its first token, and all rows of a stage past the end, are
  // zeroed by the lanes that copied them.
  template <int K>
  __device__ __forceinline__ void land(int q) const {
    // s_waitcnt vmcnt((kNB - 2) stages x 8 copies) lgkmcnt(0): fields
    // vmcnt[3:0], expcnt[6:4] (7 = no wait), lgkmcnt[11:8], vmcnt[5:4] at [15:14]
    constexpr int vm = (kNB - 2) * 2 * kUnitsPerLane;
    static_assert(vm < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((vm & 15) | ((vm >> 4) << 14) | 0x70);
    const int dup = q < nstage ? static_cast<int>(tok_begin + int64_t(q) * kKT - origin_token(q)) : kKT;
    const int lane = threadIdx.x & 63;
    uint4* dst = ring<K>() + wave * (kUnitsPerLane * 64);
#pragma unroll
    for (int i = 0; i < kUnitsPerLane; ++i) {
      if (((wave * (kUnitsPerLane * 64) + i * 64 + lane) >> 5) < dup) {
        dst[i * 64 + lane] = make_uint4(0, 0, 0, 0);
        dst[kPanelUnits + i * 64 + lane] = make_uint4(0, 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
    barrier();
  }
};

// One stage of the ring kernel: stage s in buffer K, its first k-step's
// fragments already in f0. Straight-line code: the refill, the barrier and
// the next stage's first reads run even past the last stage (on zeroed
// copies), so that the MFMA sequence has no branches.
template <int K>
__device__ __forceinline__ void ring_step(const Ring& r, int s, Frags& f0, Frags& f1, f32x16 (&acc)[4][4]) {
  constexpr int KN = (K + 1) % kNB;
  read_frags(reinterpret_cast<const char*>(ring<K>()), 1, r.oa, r.ob, f1);
  mfma_rows(f0, 0, 4, acc);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  mfma_rows(f1, 0, 2, acc);
  // keep the wait and barrier after all MFMAs that precede them
  __builtin_amdgcn_sched_barrier(0);
  r.land<KN>(s + 1);
  __builtin_amdgcn_sched_barrier(0);
  // every wave is past its reads of stage s: refill its buffer with stage s + kNB
  r.issue<K>(s + kNB);
  read_frags(reinterpret_cast<const char*>(ring<KN>()), 0, r.oa, r.ob, f0);
  mfma_rows(f1, 2, 4, acc);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
}

// The kNB stages of one trip around the ring.
template <int... K>
__device__ __forceinline__ void ring_round(const Ring& r, int s, Frags& f0, Frags& f1, f32x16 (&acc)[4][4],
                                           std::integer_sequence<int, K...>) {
  (ring_step<K>(r, s + K, f0, f1, acc), ...);
}

template <int... K>
__device__ __forceinline__ void issue_first(const Ring& r, std::integer_sequence<int, K...>) {
  (r.issue<K>(K), ...);
}

// Writes a wave's 128 x 128 float32 accumulators into the partial tile.
// D[i][j] of a 32 x 32 block: lane l, register r -> i = 8 (r / 4) + 4 (l / 32) + r % 4, j = l % 32.
__device__ __forceinline__ void store_acc(const f32x16 (&acc)[4][4], float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wi = wave >> 1, wj = wave & 1;
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

// Work item of blockIdx.x; workgroups are dispatched round robin over the
// 8 XCDs, XCD x = blockIdx % 8. With gsz == 0 (at least 8 slices), XCD x runs
// every tile of slices x, x + 8, ... in turn, so each slice streams through
// one L2 only. Otherwise XCD x runs tile group x (gsz tiles of the blocked
// order) of each slice in turn. Returns false past the end.
__device__ __forceinline__ bool work_item(int ntiles, int nsl, int gsz, const int* __restrict__ order, int& sl,
                                          int& tile) {
  const int local = blockIdx.x / kXcds, xcd = blockIdx.x % kXcds;
  int rank;
  if (gsz == 0) {
    sl = xcd + kXcds * (local / ntiles);
    rank = local % ntiles;
  } else {
    sl = local / gsz;
    rank = xcd * gsz + local % gsz;
  }
  if (sl >= nsl || rank >= ntiles) return false;
  tile = order[rank];
  return true;
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

// Ring kernel: needs 16-byte aligned rows (lda, d multiples of 8, A aligned)
// and rows >= 32.
__global__ __launch_bounds__(kThreads, 1) void syrk_partial(
    const uint16_t* __restrict__ a, int64_t lda, int64_t d, int64_t rows, int ntiles, int slice0,
    int nsl, int gsz, const int* __restrict__ order, float* __restrict__ part) {
  int sl, tile;
  if (!work_item(ntiles, nsl, gsz, order, sl, tile)) return;
  int I, J;
  tri(tile, I, J);
  Ring r;
  r.a = reinterpret_cast<const char*>(a);
  r.lda2 = lda * 2;
  r.tok_begin = int64_t(slice0 + sl) * kSlice;
  r.tok_end = r.tok_begin + kSlice < rows ? r.tok_begin + kSlice : rows;
  r.nstage = static_cast<int>((r.tok_end - r.tok_begin + kKT - 1) / kKT);
  r.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wi = r.wave >> 1, wj = r.wave & 1;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    r.oa[x] = tr_offset(wi * 128 + x * 32);
    r.ob[x] = tr_offset(wj * 128 + x * 32) + kPanelBytes;
  }
  dma_offsets(lda, d, int64_t(I) * kT, r.da);
  dma_offsets(lda, d, int64_t(J) * kT, r.db);

  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};

  // prologue: stages 0 .. kNB - 1 issued, stage 0 landed, its first fragments read
  issue_first(r, std::make_integer_sequence<int, kNB - 1>{});
  r.land<0>(0);
  r.issue<kNB - 1>(kNB - 1);
  Frags f0, f1;
  read_frags(reinterpret_cast<const char*>(ring<0>()), 0, r.oa, r.ob, f0);

  // whole rings only: stages past nstage are zero and add nothing
  for (int s = 0; s < r.nstage; s += kNB) ring_round(r, s, f0, f1, acc, std::make_integer_sequence<int, kNB>{});
  // no copy may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);
  store_acc(acc, part + (int64_t(sl) * ntiles + tile) * (kT * kT));
}

// Register-staged copy of one panel stage with zero fill for tokens >=
// tok_end and channels >= d (any alignment).
__device__ __forceinline__ void load_stage_regs(const uint16_t* __restrict__ a, int64_t lda, int64_t d, int64_t c0,
                                                int64_t t0, int64_t tok_end, uint4* __restrict__ panel) {
#pragma unroll
  for (int i = 0; i < kUnitsPerLane; ++i) {
    const int sl = i * kThreads + static_cast<int>(threadIdx.x);
    const int t = sl >> 5, cs = sl & 31;
    const int cc = (cs & 16) | ((cs & 15) ^ ((t & 3) << 2));
    const int64_t ch = c0 + int64_t(cc) * 8;
    const int64_t tok = t0 + t;
    uint32_t e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = (tok < tok_end && ch + k < d) ? a[tok * lda + ch + k] : 0u;
    panel[sl] = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
  }
}

// Fallback for unaligned rows or fewer than 32 rows: two register-staged
// buffers, one full barrier per stage.
__global__ __launch_bounds__(kThreads, 1) void syrk_partial_regs(
    const uint16_t* __restrict__ a, int64_t lda, int64_t d, int64_t rows, int ntiles, int slice0,
    int nsl, int gsz, const int* __restrict__ order, float* __restrict__ part) {
  __shared__ uint4 lds[2][2 * kPanelUnits];
  int sl, tile;
  if (!work_item(ntiles, nsl, gsz, order, sl, tile)) return;
  int I, J;
  tri(tile, I, J);
  const bool two = (I != J);
  const int64_t tok_begin = int64_t(slice0 + sl) * kSlice;
  const int64_t tok_end = tok_begin + kSlice < rows ? tok_begin + kSlice : rows;
  const int nstage = static_cast<int>((tok_end - tok_begin + kKT - 1) / kKT);
  const int wave = threadIdx.x >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  int32_t oa[4], ob[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    oa[x] = tr_offset(wi * 128 + x * 32);
    ob[x] = tr_offset(wj * 128 + x * 32) + (two ? kPanelBytes : 0);
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};
  for (int s = 0; s < nstage; ++s) {
    uint4* buf = lds[s & 1];
    const int64_t t0 = tok_begin + int64_t(s) * kKT;
    load_stage_regs(a, lda, d, int64_t(I) * kT, t0, tok_end, buf);
    if (two) load_stage_regs(a, lda, d, int64_t(J) * kT, t0, tok_end, buf + kPanelUnits);
    __syncthreads();
    Frags f;
#pragma unroll
    for (int kk = 0; kk < kKT / 16; ++kk) {
      read_frags(reinterpret_cast<const char*>(buf), kk, oa, ob, f);
      mfma_rows(f, 0, 4, acc);
    }
  }
  store_acc(acc, part + (int64_t(sl) * ntiles + tile) * (kT * kT));
}

// Sums the float32 partials of a tile in float64; at the last slice group
// writes H = alpha * S + beta * H to both triangles. One workgroup per 64 x 64
// sub-block; a thread owns 4 columns x 4 rows (16-byte loads), slices summed
// four at a time.
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
  const int cq = (threadIdx.x & 15) * 4;      // first of this thread's 4 columns
  const int rb = threadIdx.x >> 4;            // rows rb, rb + 16, rb + 32, rb + 48
  const int64_t tile_off = int64_t(tile) * kT * kT;
  const int64_t slice_stride = int64_t(ntiles) * kT * kT;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int il = rb + 16 * k;
    const int64_t e = int64_t(si * 64 + il) * kT + sj * 64 + cq;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    if (!first) {
      s0 = acc[tile_off + e];
      s1 = acc[tile_off + e + 1];
      s2 = acc[tile_off + e + 2];
      s3 = acc[tile_off + e + 3];
    }
    const float* pp = part + tile_off + e;
    int q = 0;
    for (; q + 4 <= nsl; q += 4) {
      const float4 v0 = *reinterpret_cast<const float4*>(pp + (q + 0) * slice_stride);
      const float4 v1 = *reinterpret_cast<const float4*>(pp + (q + 1) * slice_stride);
      const float4 v2 = *reinterpret_cast<const float4*>(pp + (q + 2) * slice_stride);
      const float4 v3 = *reinterpret_cast<const float4*>(pp + (q + 3) * slice_stride);
      s0 += (double(v0.x) + double(v1.x)) + (double(v2.x) + double(v3.x));
      s1 += (double(v0.y) + double(v1.y)) + (double(v2.y) + double(v3.y));
      s2 += (double(v0.z) + double(v1.z)) + (double(v2.z) + double(v3.z));
      s3 += (double(v0.w) + double(v1.w)) + (double(v2.w) + double(v3.w));
    }
    for (; q < nsl; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(pp + q * slice_stride);
      s0 += v.x;
      s1 += v.y;
      s2 += v.z;
      s3 += v.w;
    }
    if (!last) {
      acc[tile_off + e] = s0;
      acc[tile_off + e + 1] = s1;
      acc[tile_off + e + 2] = s2;
      acc[tile_off + e + 3] = s3;
      continue;
    }
    const double sv[4] = {s0, s1, s2, s3};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int jl = cq + c;
      const int64_t gi = r0 + il, gj = c0 + jl;
      double v = static_cast<double>(alpha) * sv[c];
      if (beta != 0.0f && gi < d && gj < d && (!dsub || il >= jl))
        v += static_cast<double>(beta) * static_cast<double>(h[gi * d + gj]);
      tr[il][jl] = static_cast<float>(v);
    }
  }
  if (!last) return;
  __syncthreads();
  const int jl = threadIdx.x & 63;
  const int ib = (threadIdx.x >> 6) * 16;
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
    const int al = ib + k;
    const int bl = jl;
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
  // The DMA ring copies whole 16-byte chunks of aligned rows, addresses a
  // stage with 32-bit byte offsets, and shifts a partial last stage back
  // inside A (needs 32 rows).
  const bool ring_ok = (lda % 8 == 0) && (d % 8 == 0) && (reinterpret_cast<uintptr_t>(a) % 16 == 0) &&
                       rows >= kKT && int64_t(kKT) * lda * 2 < (int64_t(1) << 31);
  {
    LaunchTimer timer("tile_order_kernel", st);
    hipLaunchKernelGGL(tile_order_kernel, dim3(1), dim3(64), 0, st, p.nt, order);
  }
  kq_status s0 = check_launch("tile_order_kernel");
  if (s0 != KQ_OK) return s0;
  for (int g = 0; g < p.ngroups; ++g) {
    const int s0 = g * p.group;
    const int nsl = (s0 + p.group <= p.nslices) ? p.group : p.nslices - s0;
    // whole slices per XCD when there are enough of them, else tile groups
    const int gsz = nsl >= kXcds ? 0 : (p.ntiles + kXcds - 1) / kXcds;
    const int per_xcd = gsz == 0 ? p.ntiles * ((nsl + kXcds - 1) / kXcds) : gsz * nsl;
    const char* kname = ring_ok ? "syrk_partial" : "syrk_partial_regs";
    {
      LaunchTimer timer(kname, st);
      hipLaunchKernelGGL(ring_ok ? syrk_partial : syrk_partial_regs, dim3(static_cast<unsigned>(per_xcd * kXcds)),
                         dim3(kThreads), 0, st, a, lda, d, rows, p.ntiles, s0, nsl, gsz, order, part);
    }
    kq_status s = check_launch(kname);
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
