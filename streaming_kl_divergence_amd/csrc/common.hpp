// Shared device helpers for the attention-KL kernels on gfx950 (CDNA4).
//
// Tiles of K (or Q) rows live in LDS as rows of 16-byte chunks.  A chunk's
// slot inside its row is XOR-swizzled with a function of the row index that
// serves both read patterns of the kernels (64 banks of 4 bytes):
//   * MFMA operand reads (one 16-byte chunk per lane, rows r .. r+15 at the
//     same logical chunk, 16 lanes per LDS cycle): 16 distinct banks groups;
//   * transposing reads (ds_read_b64_tr_b16, 32 lanes per cycle: four
//     consecutive rows times one aligned quad of chunks): the four rows land
//     on four different quads, so the 32 lanes touch all 64 banks once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SKL_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maxima start here instead of -inf: finite, so (m_old - m_new) * c
// stays a number even when the scale (and so c) is zero.
constexpr float kMaxInit = -1.0e30f;

// Row geometry of a [rows, D] tile of element type T.
template <typename T, int D>
struct Geom {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
  static constexpr int kGroups = kChunks / 2;             // chunk pairs (one per lane half)
  static_assert(kChunks >= 8, "rows must be at least 128 bytes");
};

// Swizzle of row `row` (XORed into the chunk index):
//   rows of 16+ chunks (256+ bytes, every row starts at bank 0):
//     4 * (row mod 4) + (row / 4) mod 4   - quad index moves with row mod 4,
//     position inside the quad with row / 4;
//   rows of 8 chunks (128 bytes, odd rows use the other 32 banks):
//     4 * ((row / 2) mod 2) + (row / 4) mod 4.
template <int kChunks>
__device__ __forceinline__ int row_swizzle(int row) {
  if constexpr (kChunks >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Byte offset of chunk `c` of tile row `row` inside an LDS tile.
template <typename T, int D>
__device__ __forceinline__ int lds_chunk_off(int row, int c) {
  using G = Geom<T, D>;
  return (row * G::kChunks + (c ^ row_swizzle<G::kChunks>(row))) * 16;
}

// Offsets of the MFMA operand reads in closed form.  The swizzle depends only
// on row mod 16 and XORs the chunk index, and row bits and chunk bits of an
// offset never overlap, so for r0 a multiple of 16
//   lds_chunk_off(r0 + col, 2 g + h) = (pair_base ^ 32 g) + r0 * row_bytes,
//   pair_base = lds_chunk_off(col, h).
// One per-lane base serves every row block and chunk pair: each read costs
// one XOR-add, and the row block and the tile's place in LDS become the
// instruction's immediate offset.
template <typename T, int D>
__device__ __forceinline__ int pair_base(int col, int h) { return lds_chunk_off<T, D>(col, h); }
__device__ __forceinline__ int pair_off(int base, int g) { return base ^ (32 * g); }

// acc(32 x 32) += A(32 x k) B(k x 32) for one chunk pair.  Lane l supplies one
// 16-byte chunk of row (l % 32) of A and of column (l % 32) of B; lanes l and
// l + 32 hold the two chunks of the pair.  Any fixed assignment of a row's
// elements to k works as long as A and B use the same one, so chunks can be
// read straight from row-major memory.
//   bf16: one v_mfma_f32_32x32x16_bf16 (8 elements per lane);
//   fp32: four v_mfma_f32_32x32x2_f32  (1 element per lane each).
// Result layout (both): lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4,
// column l % 32.
template <typename T>
__device__ __forceinline__ f32x16 mfma_chunk(u32x4 a, u32x4 b, f32x16 acc);

template <>
__device__ __forceinline__ f32x16 mfma_chunk<__bf16>(u32x4 a, u32x4 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma_chunk<float>(u32x4 a, u32x4 b, f32x16 acc) {
  const f32x4 fa = __builtin_bit_cast(f32x4, a);
  const f32x4 fb = __builtin_bit_cast(f32x4, b);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.x, fb.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.y, fb.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.z, fb.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.w, fb.w, acc, 0, 0, 0);
  return acc;
}

// Launch order -> work order.  The hardware deals workgroups round-robin over
// the XCDs (launch index i runs on XCD i mod 8).  Work items (head, block)
// are numbered head-major, and XCD x takes the contiguous range
// [x * per, (x + 1) * per) of them in order, so the workgroups resident on an
// XCD at any time belong to one head and stream the same key (or query) tiles
// through that XCD's L2.  The grid has kXcds * per workgroups; a returned
// index >= total marks a workgroup with nothing to do.
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_grid(int total) { return kXcds * ((total + kXcds - 1) / kXcds); }
__device__ __forceinline__ int xcd_work_index(int bid, int total) {
  const int per = (total + kXcds - 1) / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

// Row index (within a 32 x 32 MFMA result block) of register r in lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One 16-byte-per-lane copy from global memory straight into LDS
// (global_load_lds_dwordx4): lane i's 16 bytes land at lds_base + 16 * i.
// Written as inline assembly on purpose: when the compiler sees an LDS DMA in
// flight it waits for every LDS read with lgkmcnt(0), which stalls each MFMA
// for a full LDS latency.  LDS reads complete in order among themselves, so
// waiting for "at most the reads issued after mine" is correct whether or
// not the DMA is counted too (it can only raise the count).  Completion of
// the DMA itself is ordered by wait_async_loads() and a barrier before any
// wave reads the tile.  SALU writes to M0 need one wait state before an LDS
// DMA, hence the s_nop.
// NT marks the load non-temporal (the nt cache-policy bit): for data that no
// other workgroup will read again, HBM streams it faster.
template <bool NT = false>
__device__ __forceinline__ void lds_dma_16(const void* src, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off nt"
        :
        : "v"(src), "s"(lds_base)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(src), "s"(lds_base)
        : "memory", "m0");
}

// Issue the asynchronous copy of a [BK, D] tile (rows key0 .. key0+BK-1 of the
// head whose row 0 is at `g`) into LDS with the swizzled layout.  Rows past
// n_rows are clamped to the last row, so every load is in bounds; the caller
// masks those rows out.  Every lane of all NW waves takes part.
template <typename T, int D, int BK, int NW, bool NT = false>
__device__ __forceinline__ void issue_tile_async(const char* __restrict__ g, int key0, int n_rows,
                                                 SKL_LDS char* tile, int tid, int wave) {
  using G = Geom<T, D>;
  constexpr int kSlots = BK * G::kChunks;
  static_assert(kSlots % (NW * 64) == 0, "tile must split evenly over the workgroup");
  constexpr int kPer = kSlots / (NW * 64);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int slot = i * NW * 64 + tid;
    const int row = slot / G::kChunks;
    const int pc = slot % G::kChunks;
    const int c = pc ^ row_swizzle<G::kChunks>(row);
    const int src_row = min(key0 + row, n_rows - 1);
    const char* src = g + (size_t)src_row * G::kRowBytes + c * 16;
    // lane i of this wave lands at base + 16 * i
    lds_dma_16<NT>(src, __builtin_amdgcn_readfirstlane(
                        (uint32_t)(uintptr_t)(tile + (i * NW * 64 + wave * 64) * 16)));
  }
}

// The same copy in scalar-base form: a wave-uniform 64-bit base (SGPRs) plus a
// 32-bit per-lane byte offset, so a tile that needs no clamping costs no
// per-lane 64-bit address arithmetic.
template <bool NT = false>
__device__ __forceinline__ void lds_dma_16_sbase(const char* base, uint32_t voff, uint32_t lds_base) {
  // the base is wave-uniform by construction; make that visible to the
  // compiler so it stays in SGPRs
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const char* sbase = (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(sbase), "s"(lds_base)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(lds_base)
        : "memory", "m0");
}

// Streams [BK, D] tiles of one head's rows into swizzled LDS tiles.  Each
// lane's source offset inside a tile is fixed for the whole kernel, so it is
// computed once; a full tile is then one scalar base per instruction.  A tile
// that reaches past n_rows (the last one) takes the clamped path.  NT: the
// loads are non-temporal (see lds_dma_16).
template <typename T, int D, int BK, int NW, bool NT = false>
struct TileStream {
  using G = Geom<T, D>;
  static constexpr int kSlots = BK * G::kChunks;
  static_assert(kSlots % (NW * 64) == 0, "tile must split evenly over the workgroup");
  static constexpr int kPer = kSlots / (NW * 64);
  static constexpr int kRowsPerInst = NW * 64 / G::kChunks;
  // the swizzle repeats every 16 rows, so when every instruction covers a
  // multiple of 16 rows all instructions share one lane offset
  static constexpr bool kPeriodic = kRowsPerInst % 16 == 0;
  uint32_t voff0;

  __device__ __forceinline__ static uint32_t lane_off(int i, int tid) {
    const int slot = i * NW * 64 + tid;
    const int row = slot / G::kChunks;
    const int c = (slot % G::kChunks) ^ row_swizzle<G::kChunks>(row);
    return (uint32_t)(row * G::kRowBytes + c * 16);
  }
  __device__ __forceinline__ void init(int tid) { voff0 = lane_off(0, tid); }

  __device__ __forceinline__ void issue_full(const char* __restrict__ g, int key0, SKL_LDS char* tile, int tid,
                                             int wave) const {
    const char* base = g + (size_t)key0 * G::kRowBytes;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t lb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + (i * NW * 64 + wave * 64) * 16));
      if constexpr (kPeriodic)
        lds_dma_16_sbase<NT>(base + i * kRowsPerInst * G::kRowBytes, voff0, lb);
      else
        lds_dma_16_sbase<NT>(base, lane_off(i, tid), lb);
    }
  }

  __device__ __forceinline__ void issue(const char* __restrict__ g, int key0, int n_rows, SKL_LDS char* tile,
                                        int tid, int wave) const {
    if (key0 + BK > n_rows) {
      issue_tile_async<T, D, BK, NW, NT>(g, key0, n_rows, tile, tid, wave);
      return;
    }
    issue_full(g, key0, tile, tid, wave);
  }

  // The same rows of two tensors (K1 and K2, or Q1 and Q2) into two tiles,
  // under one test for the clamped last tile, so that the clamped path's
  // per-lane address work stays inside that (rare) branch.
  __device__ __forceinline__ void issue2(const char* __restrict__ g1, const char* __restrict__ g2, int key0,
                                         int n_rows, SKL_LDS char* tile1, SKL_LDS char* tile2, int tid,
                                         int wave) const {
    if (__builtin_expect(key0 + BK > n_rows, 0)) {
      issue_tile_async<T, D, BK, NW, NT>(g1, key0, n_rows, tile1, tid, wave);
      issue_tile_async<T, D, BK, NW, NT>(g2, key0, n_rows, tile2, tid, wave);
      return;
    }
    issue_full(g1, key0, tile1, tid, wave);
    issue_full(g2, key0, tile2, tid, wave);
  }
};

// Scheduling pattern for a run of N MFMAs that each take one operand from
// LDS: issue the first AHEAD reads, then alternate one MFMA with one read, so
// AHEAD reads are always in flight and no MFMA waits a full LDS latency.
// (Masks: 0x008 MFMA, 0x100 DS read.)
template <int N, int AHEAD>
__device__ __forceinline__ void sched_lds_mfma_pipeline() {
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// Wait for every outstanding scalar load (kernel arguments).  Scalar loads
// complete out of order, so while one is pending the compiler can only wait
// for LDS reads with lgkmcnt(0); after this it counts LDS reads precisely.
__device__ __forceinline__ void settle_scalar_loads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait for every outstanding vector-memory load, the LDS DMAs included.  This
// is the s_waitcnt builtin (vmcnt 0, other counters untouched; gfx9 encoding)
// rather than inline assembly on purpose: the compiler then knows that every
// earlier load has landed.  Without that it keeps waits for the register
// fragments loaded before the tile loop inside the loop, and since the
// hardware counter also holds the DMA of the next tile (issued by inline
// assembly the compiler cannot see), those waits stall every tile until its
// prefetch has arrived.
__device__ __forceinline__ void wait_async_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposing LDS read (bf16 tiles): lane l of each 16-lane group passes the
// address of element (r0 + (l % 16) / 4, c0 + 4 * (l % 4)) of a row-major
// tile and receives the four elements (r0 + e, c0 + l % 16), e = 0..3: four
// consecutive rows of one column.  (Measured lane semantics of
// ds_read_b64_tr_b16 on gfx950: result[i][e] = loaded[4e + i/4][i % 4]
// within each group of 16 lanes.)
template <int D>
__device__ __forceinline__ int tr4_off(int r0, int c0, int lane) {
  const int l16 = lane & 15;
  const int row = r0 + (l16 >> 2);
  const int cc = c0 + 4 * (l16 & 3);            // bf16 element column
  return lds_chunk_off<__bf16, D>(row, cc >> 3) + (cc & 7) * 2;
}
__device__ __forceinline__ u32x2 read_tr4_at(const SKL_LDS char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SKL_LDS s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// The transposing reads of one 32 x 32 block in closed form, as for pair_base:
// lane l reads rows rb + 16 t + 4 (l / 32) + 8 hi + (l % 16) / 4 (t, hi = 0, 1)
// at element column 32 db + 16 ((l / 16) % 2) + 4 (l % 4); for rb a multiple
// of 32 the offset is (tr_base(hi) ^ 64 db) + (rb + 16 t) * row_bytes.
template <int D>
__device__ __forceinline__ int tr_base(int lane, int hi) {
  return tr4_off<D>(4 * (lane >> 5) + 8 * hi, 16 * ((lane >> 4) & 1), lane);
}

}  // namespace skl
