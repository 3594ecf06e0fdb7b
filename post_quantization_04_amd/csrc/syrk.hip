// H = alpha * A^T A + beta * H for token-major bf16 A on gfx950 bf16 MFMA.
//
// A is [rows, d]: tokens by channels, channels contiguous. The contraction
// runs over tokens, so each MFMA operand needs consecutive tokens of one
// channel per lane. Panels of 32 tokens x 256 channels are staged in LDS in
// their natural token-major layout and the MFMA fragments are read with the
// gfx950 transposing LDS load ds_read_b64_tr_b16: in each group of 16 lanes,
// four lanes per token supply 16 consecutive channels and lane j receives
// channel j at the four tokens. Two such loads give the eight tokens of a
// v_mfma_f32_32x32x16_bf16 operand. The 16-byte chunks of each 512-byte token
// row are XOR-swizzled with the token index so that both the LDS writes and
// the transposing reads run at the LDS bank minimum.
//
// Staging: each lane loads its 16-byte chunks of a stage (both panels) into
// registers with buffer loads, three stages ahead, and writes them to LDS with
// ds_write_b128; three LDS stage buffers rotate with the three register sets.
// The buffer resource of a stage ends at the slice's last token, so rows past
// it (a partial last stage) load as zeros with no extra code. Measured against
// copying global -> LDS directly (global_load_lds_dwordx4) on the 262144 x
// 4096 covariance: 3.93 vs 4.37 ms per launch, exact same sums.
//
// Schedule of one stage (one barrier): first half, the 16 MFMAs of the
// stage's first 16-token k-step with the 16 transposing reads of its second
// k-step and the second half of the next stage's LDS writes; barrier; second
// half, the 16 MFMAs of the second k-step with the reads of the next stage's
// first k-step, the first half of the stage after next's writes and the loads
// refilling the register set just written. One MFMA per LDS read throughout,
// one LDS write per four MFMAs, so the LDS traffic is even over the stage.
//
// Diagonal tiles (I = J) load their one panel once and read both operands from
// it; the wave whose 128 x 128 block lies above the diagonal only helps stage
// the panel (that block is never read).
//
// Work item = (lower-triangle 256 x 256 output tile, token slice of 16384
// rows). Each workgroup sums one slice in float32 MFMA accumulators (bf16
// products are exact) and writes the float32 partial tile. A second kernel
// adds the slices of a tile in float64, applies alpha and beta, rounds once to
// float32 and writes both triangles. Short float32 runs (1024 roundings per
// accumulator) keep the accumulated rounding at a few 1e-7 relative, which the
// downstream column sweep needs; longer slices would write and re-read fewer
// partial tiles (16384 rather than 8192 rows: half the partial bytes, and a
// step 3 % faster on the LLaMA-2-7B q_proj covariances).
//
// Workgroups are dispatched round robin over the 8 XCDs. With at least 8
// slices, XCD x runs every tile of slices x, x + 8, ..., tiles in a blocked
// order (4 tile rows x 8 tile columns, so the 32 workgroups of an XCD share
// about 12 channel panels) and each token slice streams through one L2 only.
// With fewer slices (wide H: a launch holds one or two slices), the tiles go
// in super-blocks of 16 x 16: the 8 XCDs run one super-block together, XCD x
// its 4 x 8 sub-block x, so the 32 panels of a super-block come from HBM about
// once and reach the other XCDs from the Infinity Cache. At width 28672 this
// ran 3.5 % faster than giving each XCD a contiguous eighth of the tiles.
#include <cstdlib>
#include <utility>

#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kT = 256;          // output tile edge (channels)
constexpr int kKT = 32;          // tokens per LDS stage
constexpr int kNS = 3;           // register sets = LDS stage buffers = unroll period
constexpr int kSlice = 16384;    // tokens per float32 partial sum
constexpr int kThreads = 256;    // 4 waves in a 2 x 2 grid, 128 x 128 outputs each
constexpr int kPanelUnits = kT * kKT * 2 / 16;  // 16-byte units per LDS panel (1024)
constexpr int kPanelBytes = kPanelUnits * 16;
constexpr int kUnitsPerLane = kPanelUnits / kThreads;  // 16-byte loads per lane per panel (4)
constexpr int kTargetItems = 8192;  // work items per launch before slices are split into groups
constexpr size_t kKeepAllBytes = size_t(64) << 30;  // the partials of every slice are kept below this

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
using Rsrc = __amdgpu_buffer_rsrc_t;

#define KQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// The three stage buffers (panel I, then panel J), each its own __shared__
// object so the compiler can tell the buffer being read from the ones being
// written.
__shared__ uint4 stage0[2 * kPanelUnits];
__shared__ uint4 stage1[2 * kPanelUnits];
__shared__ uint4 stage2[2 * kPanelUnits];

template <int K>
__device__ __forceinline__ uint4* stage_buf() {
  if constexpr (K % 3 == 0) return stage0;
  else if constexpr (K % 3 == 1) return stage1;
  else return stage2;
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

// Tile t of the square (CROSS: all nt x nt tiles, t = I nt + J) or of the lower triangle.
template <bool CROSS>
__device__ __forceinline__ void tile_ij(int t, int nt, int& I, int& J) {
  if constexpr (CROSS) {
    I = t / nt;
    J = t % nt;
  } else {
    tri(t, I, J);
  }
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

// Reads in the order the MFMAs need them: row block 0's operand and the four
// column blocks first.
__device__ __forceinline__ void read_frags(const char* buf, int kk, const int32_t (&oa)[4], const int32_t (&ob)[4],
                                           Frags& f) {
  f.a[0] = frag_at(buf + oa[0] + kk * 8192);
#pragma unroll
  for (int y = 0; y < 4; ++y) f.b[y] = frag_at(buf + ob[y] + kk * 8192);
#pragma unroll
  for (int x = 1; x < 4; ++x) f.a[x] = frag_at(buf + oa[x] + kk * 8192);
}

// MFMAs of one k-step: 4 row blocks x 4 column blocks.
__device__ __forceinline__ void mfma_all(const Frags& f, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
      acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[x], f.b[y], acc[x][y], 0, 0, 0);
}

// Per-lane byte offsets (from a stage's first token row) of the chunks this
// lane stages from a panel: load i of wave w fills slot w * 256 + i * 64 +
// lane, whose chunk is the un-swizzled position. Chunks past channel d re-read
// the row's last 8 channels (their outputs are discarded).
__device__ __forceinline__ void chunk_offsets(int64_t lda, int64_t d, int64_t c0, uint32_t (&off)[kUnitsPerLane]) {
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

// Workgroup barrier without the full memory drain of __syncthreads (which
// would also wait for the loads of the stages still in flight).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// One stage of both panels (one panel for a diagonal tile) in registers:
// panel I units 0..3, then panel J units 0..3.
struct RegStage {
  uint4 v[2 * kUnitsPerLane];
};

// Uniform per-workgroup state of the pipeline. DIAG: I = J, one panel. CROSS:
// panel J comes from a second matrix B (row pitch ldb2 bytes).
template <bool DIAG, bool CROSS = false>
struct Pipe {
  const char* a;        // A as bytes
  int64_t lda2;         // row pitch in bytes
  const char* b;        // B as bytes (CROSS)
  int64_t ldb2;
  int64_t tok_begin, tok_end;
  int nstage;
  int wave;
  uint32_t da[kUnitsPerLane], db[kUnitsPerLane];
  int32_t oa[4], ob[4];

  // Stage q's 32 token rows through a buffer resource that ends at tok_end:
  // rows at or past it (a partial last stage, the stages loaded past the end
  // of the slice) read as 0.
  __device__ __forceinline__ void load(int q, RegStage& r) const {
    const int64_t t0 = tok_begin + int64_t(q) * kKT;
    int64_t left = tok_end - t0;
    left = left < 0 ? 0 : (left > kKT ? kKT : left);
    const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a + t0 * lda2), static_cast<short>(0),
                                                      static_cast<int>(left * lda2), 0x00020000);
#pragma unroll
    for (int i = 0; i < kUnitsPerLane; ++i) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, da[i], 0, 0);
      r.v[i] = make_uint4(x[0], x[1], x[2], x[3]);
    }
    if constexpr (!DIAG) {
      Rsrc rb = rs;
      if constexpr (CROSS)
        rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b + t0 * ldb2), static_cast<short>(0),
                                               static_cast<int>(left * ldb2), 0x00020000);
#pragma unroll
      for (int i = 0; i < kUnitsPerLane; ++i) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rb, db[i], 0, 0);
        r.v[kUnitsPerLane + i] = make_uint4(x[0], x[1], x[2], x[3]);
      }
    }
  }
  // Half P (units 2P, 2P + 1) of the stage in r into stage buffer K.
  template <int K, int P>
  __device__ __forceinline__ void store(const RegStage& r) const {
    const int lane = threadIdx.x & 63;
    uint4* dst = stage_buf<K>() + wave * (kUnitsPerLane * 64);
#pragma unroll
    for (int i = 2 * P; i < 2 * P + 2; ++i) {
      dst[i * 64 + lane] = r.v[i];
      if constexpr (!DIAG) dst[kPanelUnits + i * 64 + lane] = r.v[kUnitsPerLane + i];
    }
  }
};

// Instruction interleave of one half stage: 16 x (MFMA, LDS read), with an
// LDS write (and, in the second half, two global loads) every 4 MFMAs (every
// 8 for a diagonal tile).
template <int G, bool DIAG, bool LOADS>
__device__ __forceinline__ void interleave() {
  // one LDS write per group: 4 writes per half stage (2 for one panel)
  constexpr int kGroups = DIAG ? 2 : 4;
  constexpr int kPer = 16 / kGroups;
#pragma unroll
  for (int i = 0; i < kGroups; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, G);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, G);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x200, 1, G);  // LDS write
    if constexpr (LOADS) __builtin_amdgcn_sched_group_barrier(0x020, 2, G);  // global load
#pragma unroll
    for (int j = 1; j < kPer; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, G);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, G);
    }
  }
}

// One stage: stage s in buffer K % 3, its first k-step's fragments in f0.
// IDLE: the wave above the diagonal of a diagonal tile, which stages data but
// computes nothing.
template <int K, bool DIAG, bool IDLE, typename PIPE>
__device__ __forceinline__ void stage_step(const PIPE& p, int s, RegStage (&regs)[kNS], Frags& f0, Frags& f1,
                                           f32x16 (&acc)[4][4]) {
  if constexpr (!IDLE) {
    read_frags(reinterpret_cast<const char*>(stage_buf<K>()), 1, p.oa, p.ob, f1);
    mfma_all(f0, acc);
  }
  p.template store<K + 1, 1>(regs[(K + 1) % kNS]);
  if constexpr (!IDLE) interleave<0, DIAG, false>();
  __builtin_amdgcn_sched_barrier(0);
  // this wave's writes of stage s + 1 and reads of stage s are done
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier();
  __builtin_amdgcn_sched_barrier(0);
  // stage s + 1 is fully written (register set (K + 1) % 3 is free again)
  p.load(s + 1 + kNS, regs[(K + 1) % kNS]);
  if constexpr (!IDLE) {
    read_frags(reinterpret_cast<const char*>(stage_buf<K + 1>()), 0, p.oa, p.ob, f0);
    mfma_all(f1, acc);
  }
  // buffer (K + 2) % 3 held stage s - 1, whose reads all finished before the barrier
  p.template store<K + 2, 0>(regs[(K + 2) % kNS]);
  if constexpr (!IDLE) interleave<1, DIAG, true>();
  __builtin_amdgcn_sched_barrier(0);
}

template <bool DIAG, bool IDLE, typename PIPE, int... K>
__device__ __forceinline__ void stage_round(const PIPE& p, int s, RegStage (&regs)[kNS], Frags& f0, Frags& f1,
                                            f32x16 (&acc)[4][4], std::integer_sequence<int, K...>) {
  (stage_step<K, DIAG, IDLE>(p, s + K, regs, f0, f1, acc), ...);
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

// The slice loop of one work item.
template <bool DIAG, bool IDLE, bool CROSS>
__device__ __forceinline__ void slice_sum(const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ b,
                                          int64_t ldb, int64_t d, int64_t tok_begin, int64_t tok_end, int I, int J,
                                          float* __restrict__ out) {
  Pipe<DIAG, CROSS> p;
  p.a = reinterpret_cast<const char*>(a);
  p.lda2 = lda * 2;
  p.b = reinterpret_cast<const char*>(b);
  p.ldb2 = ldb * 2;
  p.tok_begin = tok_begin;
  p.tok_end = tok_end;
  p.nstage = static_cast<int>((tok_end - tok_begin + kKT - 1) / kKT);
  p.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wi = p.wave >> 1, wj = p.wave & 1;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    p.oa[x] = tr_offset(wi * 128 + x * 32);
    p.ob[x] = tr_offset(wj * 128 + x * 32) + (DIAG ? 0 : kPanelBytes);
  }
  chunk_offsets(lda, d, int64_t(I) * kT, p.da);
  chunk_offsets(CROSS ? ldb : lda, d, int64_t(J) * kT, p.db);

  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};

  // prologue: stages 0, 1, 2 in register sets 0, 1, 2; stage 0 and the first
  // half of stage 1 written; set 0 refilled with stage 3
  RegStage regs[kNS];
  p.load(0, regs[0]);
  p.load(1, regs[1]);
  p.load(2, regs[2]);
  p.template store<0, 0>(regs[0]);
  p.template store<0, 1>(regs[0]);
  p.template store<1, 0>(regs[1]);
  p.load(kNS, regs[0]);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  barrier();
  Frags f0, f1;
  if constexpr (!IDLE) read_frags(reinterpret_cast<const char*>(stage_buf<0>()), 0, p.oa, p.ob, f0);
  int s = 0;
  for (; s + kNS <= p.nstage; s += kNS)
    stage_round<DIAG, IDLE>(p, s, regs, f0, f1, acc, std::make_integer_sequence<int, kNS>{});
  // the one or two stages left (uniform branches)
  if (s < p.nstage) stage_step<0, DIAG, IDLE>(p, s, regs, f0, f1, acc);
  if (s + 1 < p.nstage) stage_step<1, DIAG, IDLE>(p, s + 1, regs, f0, f1, acc);
  // no load may still be writing this wave's registers when it exits
  __builtin_amdgcn_s_waitcnt(0);
  if constexpr (!IDLE) store_acc(acc, out);
}

// Work item of blockIdx.x; workgroups are dispatched round robin over the
// 8 XCDs, XCD x = blockIdx % 8. With nsb == 0 (at least 8 slices), XCD x runs
// every tile of slices x, x + 8, ... in turn (blocked order), so each slice
// streams through one L2 only. Otherwise the slices run one after another,
// each as nsb super-blocks of 256 slots, slot 32 x + k of a super-block being
// XCD x's k-th tile. Returns false past the end and for empty slots.
__device__ __forceinline__ bool work_item(int ntiles, int nsl, int nsb, const int* __restrict__ order, int& sl,
                                          int& tile) {
  const int local = blockIdx.x / kXcds, xcd = blockIdx.x % kXcds;
  if (nsb == 0) {
    sl = xcd + kXcds * (local / ntiles);
    if (sl >= nsl) return false;
    tile = order[local % ntiles];
    return true;
  }
  sl = local / (nsb * 32);
  if (sl >= nsl) return false;
  const int l = local % (nsb * 32);
  tile = order[(l / 32) * 256 + xcd * 32 + (l % 32)];
  return tile >= 0;
}

// Super-block slots, one workgroup per super-block, one thread per slot.
// Super-blocks of 16 x 16 tiles cover the lower triangle, row-major over the
// super-blocks (super-block b = bi (bi + 1) / 2 + bj). Position t of a
// super-block in sub-block order is tile row 16 bi + 4 (x / 2) + k / 8, tile
// column 16 bj + 8 (x % 2) + k % 8 with x = t / 32, k = t % 32: sub-block x,
// row-major inside it. A full super-block puts position t in slot t, so XCD x
// gets sub-block x; a partial one (on the diagonal or at the edge) deals its
// n tiles out in that order, ceil(n / 8) per XCD (the q-th tile to slot
// 32 (q / per) + q % per, q from a prefix count). Empty slots hold -1.
// CROSS: super-blocks cover the whole square, b = bi side + bj, and tile (i, j) is i nt + j.
template <bool CROSS>
__global__ __launch_bounds__(256) void superblock_order_kernel(int nt, int* __restrict__ slots) {
  __shared__ int cnt[256];
  int bi, bj;
  if constexpr (CROSS) {
    const int side = (nt + 15) / 16;
    bi = static_cast<int>(blockIdx.x) / side;
    bj = static_cast<int>(blockIdx.x) % side;
  } else {
    tri(static_cast<int>(blockIdx.x), bi, bj);
  }
  const int t = static_cast<int>(threadIdx.x);
  const int x = t >> 5, k = t & 31;
  const int i = 16 * bi + 4 * (x >> 1) + (k >> 3), j = 16 * bj + 8 * (x & 1) + (k & 7);
  const int valid = (i < nt && j < nt && (CROSS || j <= i)) ? 1 : 0;
  int* out = slots + size_t(blockIdx.x) * 256;
  out[t] = -1;
  // inclusive prefix count of the valid positions
  cnt[t] = valid;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = t >= o ? cnt[t - o] : 0;
    __syncthreads();
    cnt[t] += v;
    __syncthreads();
  }
  const int n = cnt[255], q = cnt[t] - valid;
  const int per = n == 256 ? 32 : (n + 7) / 8;
  if (valid) out[(q / per) * 32 + q % per] = CROSS ? i * nt + j : i * (i + 1) / 2 + j;
}

// Every lower-triangle tile in blocks of 4 tile rows x 8 tile columns,
// row-major inside a block (32 consecutive items share about 12 channel
// panels). One thread; used by launches of at least 8 slices, where H has at
// most about a thousand tiles.
// CROSS: every tile of the square, the same blocks.
template <bool CROSS>
__global__ void blocked_order_kernel(int nt, int* __restrict__ order) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int r = 0;
  for (int bi = 0; bi < nt; bi += 4)
    for (int bj = 0; bj < nt && (CROSS || bj <= bi + 3); bj += 8)
      for (int i = bi; i < bi + 4 && i < nt; ++i)
        for (int j = bj; j < bj + 8 && j < nt && (CROSS || j <= i); ++j) order[r++] = CROSS ? i * nt + j : i * (i + 1) / 2 + j;
}

// Pipelined kernel: needs 16-byte aligned rows (lda, d multiples of 8, A
// aligned; CROSS: the same of B) and 32 rows addressable with 32-bit byte
// offsets. CROSS: partial sums of A^T B over every tile of the square.
template <bool CROSS>
__global__ __launch_bounds__(kThreads, 1) void syrk_partial(
    const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ b, int64_t ldb, int64_t d,
    int64_t rows, int nt, int ntiles, int slice0, int nsl, int nsb, const int* __restrict__ order,
    float* __restrict__ part) {
  int sl, tile;
  if (!work_item(ntiles, nsl, nsb, order, sl, tile)) return;
  int I, J;
  tile_ij<CROSS>(tile, nt, I, J);
  const int64_t tok_begin = int64_t(slice0 + sl) * kSlice;
  const int64_t tok_end = tok_begin + kSlice < rows ? tok_begin + kSlice : rows;
  float* out = part + (int64_t(sl) * ntiles + tile) * (kT * kT);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (CROSS || I != J)
    slice_sum<false, false, CROSS>(a, lda, b, ldb, d, tok_begin, tok_end, I, J, out);
  else if (wave == 1)  // block (rows 0..127, columns 128..255): above the diagonal
    slice_sum<true, true, false>(a, lda, a, lda, d, tok_begin, tok_end, I, J, out);
  else
    slice_sum<true, false, false>(a, lda, a, lda, d, tok_begin, tok_end, I, J, out);
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

// Fallback for rows that are not 16-byte aligned: element loads with zero
// fill, two LDS buffers, one full barrier per stage.
template <bool CROSS>
__global__ __launch_bounds__(kThreads, 1) void syrk_partial_regs(
    const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ b, int64_t ldb, int64_t d,
    int64_t rows, int nt, int ntiles, int slice0, int nsl, int nsb, const int* __restrict__ order,
    float* __restrict__ part) {
  __shared__ uint4 lds[2][2 * kPanelUnits];
  int sl, tile;
  if (!work_item(ntiles, nsl, nsb, order, sl, tile)) return;
  int I, J;
  tile_ij<CROSS>(tile, nt, I, J);
  const bool two = CROSS || (I != J);
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
    if (two) load_stage_regs(CROSS ? b : a, CROSS ? ldb : lda, d, int64_t(J) * kT, t0, tok_end, buf + kPanelUnits);
    __syncthreads();
    Frags f;
#pragma unroll
    for (int kk = 0; kk < kKT / 16; ++kk) {
      read_frags(reinterpret_cast<const char*>(buf), kk, oa, ob, f);
      mfma_all(f, acc);
    }
  }
  store_acc(acc, part + (int64_t(sl) * ntiles + tile) * (kT * kT));
}

// Sums the float32 partials of a tile in float64; at the last slice group
// writes H = alpha * S + beta * C_in to both triangles (CROSS: C = alpha * S +
// beta * C_in over the tile only; c_in may be h). One workgroup per 64 x 64
// sub-block; a thread owns 4 columns x 4 rows (16-byte loads), slices summed
// four at a time.
template <bool CROSS>
__global__ __launch_bounds__(256) void syrk_reduce(const float* __restrict__ part, int nsl, int nt, int ntiles,
                                                   int64_t d, double* __restrict__ acc, int first,
                                                   int last, float alpha, float beta, const float* c_in,
                                                   float* h) {
  __shared__ float tr[64][65];
  const int tile = blockIdx.x >> 4;
  const int si = (blockIdx.x >> 2) & 3, sj = blockIdx.x & 3;
  int I, J;
  tile_ij<CROSS>(tile, nt, I, J);
  const bool dsub = !CROSS && (I == J) && (si == sj);  // sub-block on the diagonal of H
  if (!CROSS && I == J && sj > si) return;              // mirror of another sub-block
  const int64_t r0 = int64_t(I) * kT + si * 64, c0 = int64_t(J) * kT + sj * 64;
  const int cq = (threadIdx.x & 15) * 4;      // first of this thread's 4 columns
  const int rb = threadIdx.x >> 4;            // rows rb, rb + 16, rb + 32, rb + 48
  const int64_t tile_off = int64_t(tile) * kT * kT;
  const int64_t slice_stride = int64_t(ntiles) * kT * kT;
  // the four rows' loads of four slices at a time are all in flight together (16 per thread);
  // each entry adds its slices one by one in slice order, so the float64 total does not depend
  // on how the slices were split into launches (the running sum is stored exactly between them)
  const int64_t e0 = int64_t(si * 64 + rb) * kT + sj * 64 + cq;  // row rb; row rb + 16 k is + 16 k kT
  double sum[4][4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) sum[k][c] = 0.0;
  if (!first) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) sum[k][c] = acc[tile_off + e0 + 16 * k * kT + c];
  }
  const float* pp = part + tile_off + e0;
  int q = 0;
  for (; q + 4 <= nsl; q += 4) {
    float4 v[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[k][u] = *reinterpret_cast<const float4*>(pp + 16 * k * kT + (q + u) * slice_stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sum[k][0] += v[k][u].x;
        sum[k][1] += v[k][u].y;
        sum[k][2] += v[k][u].z;
        sum[k][3] += v[k][u].w;
      }
    }
  }
  for (; q < nsl; ++q) {
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const float4*>(pp + 16 * k * kT + q * slice_stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sum[k][0] += v[k].x;
      sum[k][1] += v[k].y;
      sum[k][2] += v[k].z;
      sum[k][3] += v[k].w;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int il = rb + 16 * k;
    if (!last) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[tile_off + e0 + 16 * k * kT + c] = sum[k][c];
      continue;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int jl = cq + c;
      const int64_t gi = r0 + il, gj = c0 + jl;
      double v = static_cast<double>(alpha) * sum[k][c];
      // CROSS rounds alpha * S to float32 first, so C_in = the same moment gives exactly 0
      if constexpr (CROSS) v = static_cast<double>(static_cast<float>(v));
      if (beta != 0.0f && gi < d && gj < d && (!dsub || il >= jl))
        v += static_cast<double>(beta) * static_cast<double>(c_in[gi * d + gj]);
      if constexpr (CROSS) {
        // each entry belongs to this tile alone: read (above) and written by the same thread
        if (gi < d && gj < d) h[gi * d + gj] = static_cast<float>(v);
      } else {
        tr[il][jl] = static_cast<float>(v);
      }
    }
  }
  if constexpr (CROSS) return;
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

// out = beta * in (0 when beta is 0); in may be out.
__global__ void scale_kernel(const float* in, float* out, int64_t n, float beta) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (beta == 0.0f) ? 0.0f : beta * in[i];
}

struct Plan {
  int nt, ntiles, nslices, group, ngroups, nsb;
  bool keep_all;  // the partials of every slice stay until one reduce after the last launch
  size_t part_bytes, acc_bytes, order_bytes;
};

// Bytes of float32 partials up to which every slice's are kept: kKeepAllBytes, or the decimal
// value of KQ_COV_KEEP_ALL_MAX_BYTES (a lower cap takes the running-sum path at small sizes).
size_t keep_all_cap() {
  const char* e = std::getenv("KQ_COV_KEEP_ALL_MAX_BYTES");
  if (e != nullptr && *e != '\0') {
    char* end = nullptr;
    const unsigned long long v = std::strtoull(e, &end, 10);
    if (end != nullptr && *end == '\0') return static_cast<size_t>(v);
  }
  return kKeepAllBytes;
}

// CROSS: every tile of the square and super-blocks over the square.
Plan plan(int64_t rows, int64_t d, bool cross) {
  Plan p{};
  p.nt = static_cast<int>((d + kT - 1) / kT);
  p.ntiles = cross ? p.nt * p.nt : p.nt * (p.nt + 1) / 2;
  p.nslices = static_cast<int>((rows + kSlice - 1) / kSlice);
  int g = (kTargetItems + p.ntiles - 1) / p.ntiles;
  if (g < 1) g = 1;
  if (g > p.nslices) g = p.nslices;
  // A launch of whole slices hands them to the XCDs one per XCD per round, so a group of
  // 8 < g < 16 slices would run a second round on g - 8 XCDs while the rest idle: groups
  // above 8 slices are cut to a multiple of 8 (the remainder forms a group of its own).
  if (g > kXcds) g -= g % kXcds;
  p.group = g;
  p.ngroups = p.nslices ? (p.nslices + g - 1) / g : 0;
  // With several launches, a float64 running sum of every tile carries the total from one
  // launch's reduce to the next: read and written once per launch. When the float32 partials of
  // all slices fit in kKeepAllBytes they are kept instead and reduced once at the end (262144
  // tokens at width 28672: 26.5 GB for H, one 5 ms reduce against eight of 1.6 ms; 52.6 GB for
  // the cross moment's full square, one reduce against sixteen that each also move the sum).
  const size_t slice_bytes = size_t(p.ntiles) * kT * kT * sizeof(float);
  p.keep_all = p.ngroups > 1 && size_t(p.nslices) * slice_bytes <= keep_all_cap();
  p.part_bytes = align_up((p.keep_all ? size_t(p.nslices) : size_t(g)) * slice_bytes, 256);
  p.acc_bytes = (p.ngroups > 1 && !p.keep_all) ? align_up(size_t(p.ntiles) * kT * kT * sizeof(double), 256) : 0;
  const int side = (p.nt + 15) / 16;
  p.nsb = cross ? side * side : side * (side + 1) / 2;  // 16 x 16 super-blocks
  p.order_bytes = align_up((size_t(p.nsb) * 256 + p.ntiles) * sizeof(int), 256);
  return p;
}

size_t workspace(int64_t rows, int64_t d, bool cross) {
  if (rows <= 0) return 0;
  const Plan p = plan(rows, d, cross);
  return p.part_bytes + p.acc_bytes + p.order_bytes;
}

// C = alpha * A^T B + beta * C_in (CROSS), or H = alpha * A^T A + beta * H (b = a, c_in = h).
template <bool CROSS>
kq_status cov_run(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, int64_t rows, int64_t d,
                  float alpha, float beta, const float* c_in, float* h, void* ws, hipStream_t st) {
  const char* kpart = CROSS ? "xcov_partial" : "syrk_partial";
  const char* kregs = CROSS ? "xcov_partial_regs" : "syrk_partial_regs";
  const char* kred = CROSS ? "xcov_reduce" : "syrk_reduce";
  if (rows == 0) {
    const int64_t n = d * d;
    {
      LaunchTimer timer("scale_kernel", st);
      hipLaunchKernelGGL(scale_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                         beta == 0.0f ? h : c_in, h, n, beta);
    }
    return check_launch("scale_kernel");
  }
  const Plan p = plan(rows, d, CROSS);
  float* part = static_cast<float*>(ws);
  double* acc = reinterpret_cast<double*>(static_cast<char*>(ws) + p.part_bytes);
  int* order = reinterpret_cast<int*>(static_cast<char*>(ws) + p.part_bytes + p.acc_bytes);
  // The pipelined kernel loads whole 16-byte chunks of aligned rows and
  // addresses a stage with 32-bit byte offsets.
  auto aligned = [&](const uint16_t* m, int64_t ld) {
    return (ld % 8 == 0) && (reinterpret_cast<uintptr_t>(m) % 16 == 0) && int64_t(kKT) * ld * 2 < (int64_t(1) << 31);
  };
  const bool pipe_ok = (d % 8 == 0) && aligned(a, lda) && (!CROSS || aligned(b, ldb));
  // whole slices per XCD (blocked order) where a launch holds at least 8 slices, else super-blocks
  // shared by the XCDs; the tile orders are built for the launches below by the same rule
  auto slices_of = [&](int g) { return (g * p.group + p.group <= p.nslices) ? p.group : p.nslices - g * p.group; };
  auto superblocks_of = [&](int nsl) { return nsl >= kXcds ? 0 : p.nsb; };
  bool need_blocked = false, need_sb = false;
  for (int g = 0; g < p.ngroups; ++g) (superblocks_of(slices_of(g)) == 0 ? need_blocked : need_sb) = true;
  if (need_sb) {
    {
      LaunchTimer timer("superblock_order_kernel", st);
      hipLaunchKernelGGL(superblock_order_kernel<CROSS>, dim3(static_cast<unsigned>(p.nsb)), dim3(256), 0, st, p.nt,
                         order);
    }
    const kq_status s0 = check_launch("superblock_order_kernel");
    if (s0 != KQ_OK) return s0;
  }
  if (need_blocked) {
    {
      LaunchTimer timer("blocked_order_kernel", st);
      hipLaunchKernelGGL(blocked_order_kernel<CROSS>, dim3(1), dim3(64), 0, st, p.nt, order + size_t(p.nsb) * 256);
    }
    const kq_status s0 = check_launch("blocked_order_kernel");
    if (s0 != KQ_OK) return s0;
  }
  for (int g = 0; g < p.ngroups; ++g) {
    const int s0 = g * p.group;
    const int nsl = slices_of(g);
    const int nsb = superblocks_of(nsl);
    const int per_xcd = nsb == 0 ? p.ntiles * ((nsl + kXcds - 1) / kXcds) : nsb * 32 * nsl;
    const int* ord = nsb == 0 ? order + size_t(p.nsb) * 256 : order;
    const char* kname = pipe_ok ? kpart : kregs;
    float* out = p.keep_all ? part + size_t(s0) * p.ntiles * kT * kT : part;
    {
      LaunchTimer timer(kname, st);
      hipLaunchKernelGGL(pipe_ok ? syrk_partial<CROSS> : syrk_partial_regs<CROSS>,
                         dim3(static_cast<unsigned>(per_xcd * kXcds)), dim3(kThreads), 0, st, a, lda, b, ldb, d, rows,
                         p.nt, p.ntiles, s0, nsl, nsb, ord, out);
    }
    kq_status s = check_launch(kname);
    if (s != KQ_OK) return s;
    if (p.keep_all && g + 1 < p.ngroups) continue;
    {
      LaunchTimer timer(kred, st);
      // keep_all: one reduce over every slice; otherwise this launch's slices onto the running sum
      hipLaunchKernelGGL(syrk_reduce<CROSS>, dim3(static_cast<unsigned>(p.ntiles * 16)), dim3(256), 0, st, part,
                         p.keep_all ? p.nslices : nsl, p.nt, p.ntiles, d, acc, (p.keep_all || g == 0) ? 1 : 0,
                         g == p.ngroups - 1 ? 1 : 0, alpha, beta, c_in, h);
    }
    s = check_launch(kred);
    if (s != KQ_OK) return s;
  }
  return KQ_OK;
}

}  // namespace

size_t syrk_workspace(int64_t rows, int64_t d) { return workspace(rows, d, false); }
size_t xcov_workspace(int64_t rows, int64_t d) { return workspace(rows, d, true); }

kq_status syrk_run(const uint16_t* a, int64_t rows, int64_t d, int64_t lda, float alpha, float beta,
                   float* h, void* ws, hipStream_t st) {
  return cov_run<false>(a, lda, a, lda, rows, d, alpha, beta, h, h, ws, st);
}

kq_status xcov_run(const uint16_t* a, const uint16_t* b, int64_t rows, int64_t d, int64_t lda, int64_t ldb,
                   float alpha, float beta, const float* c_in, float* c, void* ws, hipStream_t st) {
  return cov_run<true>(a, lda, b, ldb, rows, d, alpha, beta, c_in, c, ws, st);
}

}  // namespace kq
