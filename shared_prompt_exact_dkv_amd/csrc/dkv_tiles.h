// dkv_tiles.h -- staging of key/value (or query) tiles in LDS and operand reads.
//
// A tile is consecutive rows of one head of a token-major [rows, H, HD] tensor.  Two
// mechanisms:
//   - h16 kernels: LDS DMA (buffer loads that write LDS directly) into dense tiles
//     whose 16-byte chunks are swizzled per row (below); rows past a region's end
//     read as zeros through the buffer resource's size.
//   - fp32 kernels: 256 threads load the tile with 16-byte reads into registers (the
//     next tile's loads in flight while the current one is used) and store it to a
//     row layout padded by one word per row; rows at or beyond `nrows` are zero.
// Zero rows keep masked keys from injecting non-finite values into a product.
#pragma once

#include "dkv_device.h"
#include "dkv_launch.h"
#include "dkv_walks.h"

namespace dkv {

template <typename T, int HD, int BN> struct TileCfg;

// fp32: single-element operand reads, rows padded by one word.
template <int HD, int BN> struct TileCfg<float, HD, BN> {
  static constexpr int kRowStride = HD + 1;
  static constexpr int kRowBytes = BN * kRowStride * 4;
  static constexpr int kChunks = BN * HD / 4;
  static constexpr int kRowPasses = (kChunks + 255) / 256;
};

// Registers holding one fp32 tile in flight for the row layout.
template <typename T, int HD, int BN> struct RowRegs {
  static_assert(sizeof(T) == 4, "register-staged tiles are fp32");
  using C = TileCfg<T, HD, BN>;
  uint4 r[C::kRowPasses];

  // base: element pointer of row 0, head already applied; ld: elements per row.
  __device__ __forceinline__ void load(const T *base, long ld, int nrows, int tid) {
    constexpr int per_row = HD / 4;
#pragma unroll
    for (int p = 0; p < C::kRowPasses; ++p) {
      int id = p * 256 + tid;
      int row = id / per_row, ch = id % per_row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (id < C::kChunks && row < nrows)
        v = *reinterpret_cast<const uint4 *>(base + (long)row * ld + ch * 4);
      r[p] = v;
    }
  }

  __device__ __forceinline__ void store(char *lds, int tid) const {
    constexpr int per_row = HD / 4;
#pragma unroll
    for (int p = 0; p < C::kRowPasses; ++p) {
      int id = p * 256 + tid;
      if (id >= C::kChunks) continue;
      int row = id / per_row, ch = id % per_row;
      float *f = reinterpret_cast<float *>(lds) + row * C::kRowStride + ch * 4;
      f[0] = __uint_as_float(r[p].x);
      f[1] = __uint_as_float(r[p].y);
      f[2] = __uint_as_float(r[p].z);
      f[3] = __uint_as_float(r[p].w);
    }
  }
};

// A-operand fragment (one fp32 element) of a row-layout tile: row `row`, k-chunk `kc`.
template <typename T, int HD, int BN>
__device__ __forceinline__ float row_frag(const char *lds, int row, int kc, int half) {
  using C = TileCfg<T, HD, BN>;
  return reinterpret_cast<const float *>(lds)[row * C::kRowStride + kc * 2 + half];
}

// Single fp32 element of a row-layout tile (fp32 contraction over rows).
template <int HD, int BN>
__device__ __forceinline__ float row_elem(const char *lds, int row, int col) {
  return reinterpret_cast<const float *>(lds)[row * TileCfg<float, HD, BN>::kRowStride + col];
}

// A buffer resource over `bytes` bytes from `base`: buffer loads at offsets past the
// end return zero, which fills rows beyond the end of a region without a test.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// ------------------------------------------------------------ LDS DMA tiles --
//
// gfx950 buffer loads with the `lds` bit write each lane's 16 bytes straight to LDS
// at M0 + 16 * lane: one wave instruction fills 1 KB, with any source address per
// lane, and a lane past the end of the buffer resource writes zeros.  Tiles staged
// this way need no staging registers and no LDS store instructions.  The load is
// issued from inline assembly so that the compiler does not wait for it before every
// LDS read; the kernels wait (`dma_wait`) right before the barrier that publishes a
// stage.  M0 is saved and restored around the load.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}
// 4-byte form: lane i's word goes to M0 + 4 * i (256 bytes per wave instruction).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), issued through the
// builtin so that the compiler's own wait insertion knows every earlier vector-memory
// load has completed.  Through inline assembly it would not: it would keep loads from
// before the DMA loop (the Q fragments, say) pending and wait for them inside the loop
// with counts that, since the DMA loads of the next tile also count, stall on that
// tile's arrival.
__device__ __forceinline__ void dma_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(K) (K < 64): wait until at most the K most recently issued vector
// memory loads are outstanding (loads complete in issue order), e.g. all but the next
// stage's DMA loads.  Through the builtin, for the same reason as dma_wait.
template <int K> __device__ __forceinline__ void dma_wait_keep() {
  static_assert(K >= 0 && K < 64, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (K & 15) | ((K >> 4) << 14));
  asm volatile("" ::: "memory");
}

// A buffer resource built from values the compiler cannot prove wave-uniform (the
// callers' are uniform by construction): the operands of the DMA instructions must
// live in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u(const void *base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return make_rsrc(reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}

// LDS byte address of a pointer into __shared__ memory (the low 32 bits of its flat
// address inside the LDS aperture).
__device__ __forceinline__ uint32_t lds_u32(const void *p) { return (uint32_t)(uintptr_t)p; }

// cu[i] for a wave-uniform index, through the scalar unit (waited for on the LDS /
// scalar counter).  A vector load here would count on the vector-memory counter, and
// the wait for it would also wait for the DMA loads of the next stage in flight.
__device__ __forceinline__ int32_t sload_i32(const int32_t *base, int i) {
  const uint64_t p = (uint64_t)(uintptr_t)(base + i);
  const uint64_t pu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(pu));
  return v;
}

// 16 bytes read at a 32-bit LDS byte address.
__device__ __forceinline__ h16x8 lds_frag_at(uint32_t addr) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) const u32x4 lu32x4;
  return __builtin_bit_cast(h16x8, *(lu32x4 *)(size_t)addr);
}

// Swizzled dense tile [row][HD] h16: the 16-byte chunk c of row r sits in slot
// c ^ swz(r).  With rows of 16 or more chunks, swz(r) (bits r3 r2 r1 r0 of r) is
//   ((r0 ^ r3) << 3) | (r1 << 2) | (r0 << 1) | r2,
// a bijection on 16 consecutive rows (a 16-byte fragment read of 16 rows touches 16
// different slots), distinct in its low 3 bits over 8 rows, and distinct in bits 1-2
// and in bits 2-3 over each aligned group of 4 rows (the 4 rows of a transpose read
// land in 4 different 32- and 64-byte slot groups), so both access patterns spread
// over all banks whether the LDS serves 128 or 256 bytes per clock.  With 8-chunk
// rows the 3-bit form (r1 r0 r2) keeps the same properties for 8-row groups.
template <int HD> struct Swz {
  static constexpr int kChunks = HD / 8;   // 16-byte chunks per row
  __device__ __forceinline__ static int swz(int r) {
    const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
    if constexpr (kChunks >= 16) return ((r0 ^ r3) << 3) | (r1 << 2) | (r0 << 1) | r2;
    return (r1 << 2) | (r0 << 1) | r2;
  }
  __device__ __forceinline__ static int off(int r, int chunk) {   // byte offset of a chunk
    return r * (HD * 2) + ((chunk ^ swz(r)) << 4);
  }
};

// A-/B-operand fragment (8 h16 of one row) of a swizzled tile: row `row`, k-chunk kc.
template <int HD>
__device__ __forceinline__ h16x8 sw_frag(const char *lds, int row, int kc, int half) {
  return as_h16x8(*reinterpret_cast<const uint4 *>(lds + Swz<HD>::off(row, kc * 2 + half)));
}

// Transposed operand from a swizzled tile with the gfx950 transpose read
// (ds_read_b64_tr_b16).  Within each 16-lane group that instruction returns, in lane
// i, element k, the (i % 4)-th of the four 16-bit values addressed by lane 4k + i/4.
// Lane j of a group therefore points at row base + j/4, columns c0 + 4*(j%4) .. +3,
// and lane i receives column c0 + i of the four rows base .. base+3.  Two such reads
// give the MFMA k-operand for column col0 + lane % 32 over the 16-row slice starting
// at row0, in the kappa row order of a C tile (rows 4*half + 0..3, then
// 8 + 4*half + 0..3).
template <int HD>
__device__ __forceinline__ h16x8 sw_tr_frag(const char *lds, int row0, int col0, int lane) {
  const int half = lane >> 5, grp = (lane >> 4) & 1, j = lane & 15;
  const int col = col0 + 16 * grp + 4 * (j & 3);
  const int r1 = row0 + 4 * half + (j >> 2);
  const int inb = (col & 7) * 2;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) char lchar;
  auto p1 = reinterpret_cast<__attribute__((address_space(3))) s16x4 *>(
      (lchar *)(lds) + Swz<HD>::off(r1, col >> 3) + inb);
  auto p2 = reinterpret_cast<__attribute__((address_space(3))) s16x4 *>(
      (lchar *)(lds) + Swz<HD>::off(r1 + 8, col >> 3) + inb);
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p2);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(h16x8, r);
}

// Factored fragment addresses for swizzled tiles of HDP-wide rows (HDP = 256 or 512:
// RB = 512 or 1024 bytes per row).  In a lane's reads of one tile the swizzle XOR touches
// only chunk bits 0-3, so every read is one of 8 lane patterns (the XOR of a lane term
// with a small constant) plus an immediate offset: a tile's reads of each kind cost 8
// address operations instead of a full swizzle evaluation per read.
template <int HDP> struct SwWide {
  static constexpr int RB = HDP * 2;
  uint32_t srow;    // row-operand reads: row col, at col * RB + ((half ^ swz(col)) << 4)
  uint32_t tr[2];   // transposed reads: row 4 half + j / 4 (+ 8), 8 (j & 1) bytes in,
                    // chunk term (c_l ^ swz(row)) << 4, c_l = 2 ((lane / 16) & 1) + (j & 3) / 2
  __device__ __forceinline__ void init(int lane) {
    const int col = lane & 31, half = lane >> 5, j = lane & 15;
    const int c_l = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
    const int r = 4 * half + (j >> 2);
    srow = col * RB + ((half ^ Swz<HDP>::swz(col)) << 4);
    tr[0] = r * RB + 8 * (j & 1) + ((c_l ^ Swz<HDP>::swz(r)) << 4);
    tr[1] = r * RB + 8 * (j & 1) + ((c_l ^ Swz<HDP>::swz(r + 8)) << 4);
  }
  // Keeps the lane terms opaque to the compiler, so the 16 patterns are formed per
  // tile instead of living in registers across a loop.
  __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(srow), "+v"(tr[0]), "+v"(tr[1])); }
  // Same as sw_frag<HDP>(tile, col, kc, half) for kc >= 0 past a column base that is a
  // multiple of 128 elements (folded into `tile`).
  __device__ __forceinline__ h16x8 frag(uint32_t tile, int kc) const {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const char lchar;
    lchar *base = (lchar *)(size_t)(tile + (srow ^ ((kc & 7) << 5)));
    return __builtin_bit_cast(h16x8, *(const __attribute__((address_space(3))) u32x4 *)(base + (kc >> 3) * 256));
  }
  // Same as sw_tr_frag<HDP>(tile, row0, 32 db, lane): row0 a multiple of 16, db the
  // 32-wide column block counted from `tile`, which holds a column base that is a
  // multiple of 128 elements (or none).
  __device__ __forceinline__ h16x8 trfrag(uint32_t tile, int row0, int db) const {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 ls16x4;
    typedef __attribute__((address_space(3))) char lchar;
    const int o = row0 * RB + (db >> 2) * 256;   // immediate offsets
    lchar *b0 = (lchar *)(size_t)(tile + (tr[0] ^ ((db & 3) << 6)));
    lchar *b1 = (lchar *)(size_t)(tile + (tr[1] ^ ((db & 3) << 6)));
    s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4 *)(b0 + o));
    s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4 *)(b1 + o + 8 * RB));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(h16x8, r);
  }
};

// DMA of a ROWS x HD h16 tile of consecutive rows (row stride ld_bytes, head offset
// already in `base`) into a swizzled tile of HDP-wide rows (HDP >= HD, a power of two:
// head dims 96 and 192 are staged in 128- and 256-wide rows whose chunks past HD read as
// zeros).  Block b (1 KB) of the tile is written by wave b % 4; lane i of that
// instruction fills slot i of the block.  The per-lane source offsets depend only on
// the thread and the row stride.
template <int HDP, int ROWS, int HD = HDP> struct DmaRows {
  static_assert(HD <= HDP && HD % 8 == 0, "real head dim within the staged row");
  static constexpr int kBlocks = ROWS * HDP * 2 / 1024;
  static_assert(kBlocks % 4 == 0, "tile must be a multiple of 4 KB");
  static constexpr int kPerWave = kBlocks / 4;
  // A 1 KB block is one row at HDP = 512: the row is wave-uniform, so only the lane's
  // chunk offset is kept and the swizzle and row offset are applied per load.
  static constexpr bool kRowPerBlock = Swz<HDP>::kChunks == 64;
  static_assert(!kRowPerBlock || HD == HDP, "1 KB rows are never padded");
  static constexpr int kRegs = kRowPerBlock ? 1 : kPerWave;
  // A source offset no buffer range reaches: the lane's slot is zero-filled.
  static constexpr int kZeroOff = 0x7ffffff0;
  int voff[kRegs];
  int ld = 0, w = 0;
  __device__ __forceinline__ void init(int wave, int lane, int ld_bytes) {
    if constexpr (kRowPerBlock) {
      voff[0] = lane << 4;
      ld = ld_bytes;
      w = wave;
    } else {
#pragma unroll
      for (int k = 0; k < kPerWave; ++k) {
        const int slot = (k * 4 + wave) * 64 + lane;
        const int r = slot / Swz<HDP>::kChunks, cs = slot % Swz<HDP>::kChunks;
        const int src = cs ^ Swz<HDP>::swz(r);   // the source chunk this slot holds
        voff[k] = src < HD / 8 ? r * ld_bytes + (src << 4) : kZeroOff;
      }
    }
  }
  // nrows: valid rows from base (rows past them are zero-filled).
  __device__ __forceinline__ void load(char *lds_tile, const h16 *base, int ld_bytes, int nrows,
                                       int wave) const {
    const int n = nrows < ROWS ? (nrows > 0 ? nrows : 0) : ROWS;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc_u(base, n > 0 ? (uint32_t)((n - 1) * ld_bytes + HD * 2) : 0u);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_u32(lds_tile) + wave * 1024);
    if constexpr (kRowPerBlock) {
      const int wv = __builtin_amdgcn_readfirstlane(w);
      const int lds_ = __builtin_amdgcn_readfirstlane(ld);
#pragma unroll
      for (int k = 0; k < kPerWave; ++k) {
        const int r = k * 4 + wv;
        // The row offset stays in the vector offset: the buffer range check (which
        // zero-fills rows past nrows) covers the vector and instruction offsets only.
        dma16(rs, l0 + k * 4096, (voff[0] ^ (Swz<HDP>::swz(r) << 4)) + r * lds_);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPerWave; ++k) dma16(rs, l0 + k * 4096, voff[k]);
    }
  }
};


// ------------------------------------------------------- work-item walks --

// The walks themselves (KeyTiles, RowSteps) live in dkv_walks.h, which host code can
// include; on the device a sequence bound is read through the scalar unit.
struct ScalarCu {
  static __device__ __forceinline__ int32_t load(const int32_t *cu, int i) { return sload_i32(cu, i); }
};

}  // namespace dkv
