// dkv_tiles.h -- cooperative HBM -> LDS staging of one key/value (or query) tile.
//
// A tile is BN consecutive rows of one head of a token-major [rows, H, HD] tensor.
// 256 threads load it with 16-byte coalesced reads into registers (so the next
// tile's loads are in flight while the current tile is being used) and later store
// it to LDS in one of two layouts:
//   row layout  [row][HD + pad]      -- operand whose contraction runs over HD
//   T4 layout   [row/4][HD][row%4]   -- operand whose contraction runs over rows,
//                                       read as 4-row runs in the MFMA k order
// Rows at or beyond `nrows` are filled with zeros so that masked keys can never
// inject non-finite values into a product.
#pragma once

#include "dkv_device.h"

namespace dkv {

template <typename T, int HD, int BN> struct TileCfg;

// bf16: row layout pads each row by 16 bytes (conflict-free 16-byte reads of 32
// different rows); T4 layout needs no pad.
template <int HD, int BN> struct TileCfg<bf16, HD, BN> {
  static constexpr int kRowStride = HD + 8;                 // elements
  static constexpr int kRowBytes = BN * kRowStride * 2;
  static constexpr int kT4Bytes = BN * HD * 2;
  static constexpr int kChunks = BN * HD / 8;               // 16-byte chunks per tile
  static constexpr int kRowPasses = (kChunks + 255) / 256;
  static constexpr int kT4Tasks = (BN / 4) * (HD / 8);      // 4 rows x 8 cols each
  static constexpr int kT4Passes = (kT4Tasks + 255) / 256;
};

// fp32: single-element operand reads, rows padded by one word.
template <int HD, int BN> struct TileCfg<float, HD, BN> {
  static constexpr int kRowStride = HD + 1;
  static constexpr int kRowBytes = BN * kRowStride * 4;
  static constexpr int kT4Bytes = 0;
  static constexpr int kChunks = BN * HD / 4;
  static constexpr int kRowPasses = (kChunks + 255) / 256;
  static constexpr int kT4Tasks = 0;
  static constexpr int kT4Passes = 0;
};

// Registers holding one tile in flight for the row layout.
template <typename T, int HD, int BN> struct RowRegs {
  using C = TileCfg<T, HD, BN>;
  uint4 r[C::kRowPasses];

  // base: element pointer of row 0, head already applied; ld: elements per row.
  __device__ __forceinline__ void load(const T *base, long ld, int nrows, int tid) {
    constexpr int per_row = (sizeof(T) == 2) ? HD / 8 : HD / 4;
#pragma unroll
    for (int p = 0; p < C::kRowPasses; ++p) {
      int id = p * 256 + tid;
      int row = id / per_row, ch = id % per_row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (id < C::kChunks && row < nrows)
        v = *reinterpret_cast<const uint4 *>(base + (long)row * ld + ch * (16 / sizeof(T)));
      r[p] = v;
    }
  }

  __device__ __forceinline__ void store(char *lds, int tid) const {
    constexpr int per_row = (sizeof(T) == 2) ? HD / 8 : HD / 4;
#pragma unroll
    for (int p = 0; p < C::kRowPasses; ++p) {
      int id = p * 256 + tid;
      if (id >= C::kChunks) continue;
      int row = id / per_row, ch = id % per_row;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4 *>(lds + (row * C::kRowStride + ch * 8) * 2) = r[p];
      } else {
        float *f = reinterpret_cast<float *>(lds) + row * C::kRowStride + ch * 4;
        f[0] = __uint_as_float(r[p].x);
        f[1] = __uint_as_float(r[p].y);
        f[2] = __uint_as_float(r[p].z);
        f[3] = __uint_as_float(r[p].w);
      }
    }
  }
};

// A buffer resource over `bytes` bytes from `base`: buffer loads at offsets past the
// end return zero, which fills rows beyond the end of a region without a test.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One bf16 tile of ROWS rows x HD columns (one head of a token-major tensor) staged
// through registers into the padded row layout.  Each thread owns fixed 16-byte
// chunks, so the per-tile cost is one buffer load and one LDS store per chunk; the
// tile's base and valid length go into the (scalar) buffer resource.
template <int HD, int ROWS> struct BufRows {
  using C = TileCfg<bf16, HD, ROWS>;
  static constexpr int kPerRow = HD / 8;
  static constexpr int kPasses = C::kRowPasses;
  static_assert(C::kChunks % 256 == 0, "tile must be a whole number of 256-thread passes");
  uint4 r[kPasses];

  // Byte offset in the tensor of this thread's chunk in pass p (row stride ld_bytes).
  __device__ __forceinline__ static int goff(int p, int tid, int ld_bytes) {
    const int id = p * 256 + tid;
    return (id / kPerRow) * ld_bytes + (id % kPerRow) * 16;
  }
  __device__ __forceinline__ static int loff(int p, int tid) {
    const int id = p * 256 + tid;
    return ((id / kPerRow) * C::kRowStride + (id % kPerRow) * 8) * 2;
  }
  // base: row 0 of the tile (head offset applied); nrows: valid rows from base.
  __device__ __forceinline__ void load(const bf16 *base, int ld_bytes, int nrows, int tid) {
    const int n = nrows < ROWS ? (nrows > 0 ? nrows : 0) : ROWS;
    // The last valid row ends at its head's 16-byte chunks; rows >= n read as zero.
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, n > 0 ? (uint32_t)((n - 1) * ld_bytes + HD * 2) : 0u);
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
      r[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, goff(p, tid, ld_bytes), 0, 0));
  }
  __device__ __forceinline__ void store(char *lds, int tid) const {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) *reinterpret_cast<uint4 *>(lds + loff(p, tid)) = r[p];
  }
};

// Registers holding one bf16 tile in flight for the T4 layout.
template <int HD, int BN> struct T4Regs {
  using C = TileCfg<bf16, HD, BN>;
  uint4 r[C::kT4Passes][4];

  __device__ __forceinline__ void load(const bf16 *base, long ld, int nrows, int tid) {
#pragma unroll
    for (int p = 0; p < C::kT4Passes; ++p) {
      int id = p * 256 + tid;
      int kg = id / (HD / 8), dc = id % (HD / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int row = kg * 4 + i;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (id < C::kT4Tasks && row < nrows)
          v = *reinterpret_cast<const uint4 *>(base + (long)row * ld + dc * 8);
        r[p][i] = v;
      }
    }
  }

  __device__ __forceinline__ void store(char *lds, int tid) const {
#pragma unroll
    for (int p = 0; p < C::kT4Passes; ++p) {
      int id = p * 256 + tid;
      if (id >= C::kT4Tasks) continue;
      int kg = id / (HD / 8), dc = id % (HD / 8);
      const uint32_t *a = reinterpret_cast<const uint32_t *>(&r[p][0]);
      const uint32_t *b = reinterpret_cast<const uint32_t *>(&r[p][1]);
      const uint32_t *c = reinterpret_cast<const uint32_t *>(&r[p][2]);
      const uint32_t *d = reinterpret_cast<const uint32_t *>(&r[p][3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 lo = make_uint2(pack_lo(a[i], b[i]), pack_lo(c[i], d[i]));
        uint2 hi = make_uint2(pack_hi(a[i], b[i]), pack_hi(c[i], d[i]));
        int dim = dc * 8 + 2 * i;
        *reinterpret_cast<uint2 *>(lds + ((long)kg * HD + dim) * 8) = lo;
        *reinterpret_cast<uint2 *>(lds + ((long)kg * HD + dim + 1) * 8) = hi;
      }
    }
  }
};

// A-operand fragment of a row-layout tile: row `row`, k-chunk `kc`.
template <typename T, int HD, int BN>
__device__ __forceinline__ typename Mfma<T>::frag row_frag(const char *lds, int row, int kc,
                                                           int half) {
  using C = TileCfg<T, HD, BN>;
  if constexpr (sizeof(T) == 2) {
    uint4 u = *reinterpret_cast<const uint4 *>(lds + (row * C::kRowStride + kc * 16 + half * 8) * 2);
    return as_bf16x8(u);
  } else {
    return reinterpret_cast<const float *>(lds)[row * C::kRowStride + kc * 2 + half];
  }
}

// Operand fragment of a T4 bf16 tile for column `col` over the 16-row slice
// `slice`, in the kappa order of a C tile used as the other operand.
template <int HD>
__device__ __forceinline__ bf16x8 t4_frag(const char *lds, int slice, int col, int half) {
  int kg = slice * 4 + half;
  uint2 lo = *reinterpret_cast<const uint2 *>(lds + ((long)kg * HD + col) * 8);
  uint2 hi = *reinterpret_cast<const uint2 *>(lds + ((long)(kg + 2) * HD + col) * 8);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Single fp32 element of a row-layout tile (fp32 contraction over rows).
template <int HD, int BN>
__device__ __forceinline__ float row_elem(const char *lds, int row, int col) {
  return reinterpret_cast<const float *>(lds)[row * TileCfg<float, HD, BN>::kRowStride + col];
}

// Transposed operand straight from a row-layout bf16 tile with the gfx950
// transpose read (ds_read_b64_tr_b16).  Within each 16-lane group that
// instruction returns, in lane i, element k, the (i % 4)-th of the four 16-bit
// values addressed by lane 4k + i/4.  Lane j of a group therefore points at
// row base + j/4, columns c0 + 4*(j%4) .. +3, and lane i receives column c0 + i of
// the four rows base .. base+3.  Two such reads give the MFMA k-operand for
// column (col0 + l % 32) over the 16-row slice starting at row0, in the kappa row
// order (rows 4*half + 0..3, then 8 + 4*half + 0..3).
template <int STRIDE>
__device__ __forceinline__ bf16x8 tr_frag(const char *lds, int row0, int col0, int lane) {
  const int half = lane >> 5, grp = (lane >> 4) & 1, j = lane & 15;
  const int col = col0 + 16 * grp + 4 * (j & 3);
  const int r1 = row0 + 4 * half + (j >> 2);
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  auto p1 = reinterpret_cast<__attribute__((address_space(3))) s16x4 *>(
      (__attribute__((address_space(3))) char *)(lds) + (r1 * STRIDE + col) * 2);
  auto p2 = reinterpret_cast<__attribute__((address_space(3))) s16x4 *>(
      (__attribute__((address_space(3))) char *)(lds) + ((r1 + 8) * STRIDE + col) * 2);
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p2);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace dkv
