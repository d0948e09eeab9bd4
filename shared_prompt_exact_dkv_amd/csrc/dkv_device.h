// dkv_device.h -- device-side building blocks shared by the DualKV kernels (gfx950).
//
// Matrix products use the CDNA4 32x32 MFMA forms:
//   bf16: v_mfma_f32_32x32x16_bf16  A[32x16] * B[16x32] -> C[32x32] fp32
//   fp16: v_mfma_f32_32x32x16_f16   (same shapes and lane layout)
//   fp32: v_mfma_f32_32x32x2_f32    A[32x2]  * B[2x32]  -> C[32x32] fp32
// Lane layout (wave64, lane l, col = l % 32, half = l / 32):
//   A operand: row = col, k = half * KL + [0, KL)      (KL = 8 16-bit / 1 fp32)
//   B operand: column = col, same k split
//   C: column = col; element v (0..15) is row 8*(v/4) + 4*half + (v%4)
// So a C tile read back per lane is "one column, 16 rows"; the kernels compute
// transposed score tiles (keys x queries) so that each lane owns one query row of
// the softmax, and feed the C tile straight back as the B operand of the next
// product.  A C tile used as a k-operand pairs lane-half `half`, element e with row
//   kappa(half, e) = 8*(e/4) + 4*half + (e%4)     (within a 16-row slice)
// and the other operand is read in that same order (the transpose read of the h16
// tiles, sw_tr_frag in dkv_tiles.h; single elements in the fp32 kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dkv {

// 16-bit tensors (bf16 or fp16) are moved as h16 payloads: global rows, LDS tiles and
// MFMA fragments never look at the bits.  A 16-bit kernel's element type E (h16 itself
// for bf16, f16 for fp16) interprets them: mma16<E> runs that type's MFMA, rnd<E> /
// pack8<E> round fp32 values into payloads (nearest even) and val<E> reads a payload
// element as fp32.
typedef __bf16 h16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 h16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 h16x4;
typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

template <typename E> __device__ __forceinline__ f32x16 mma16(h16x8 a, h16x8 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mma16<h16>(h16x8 a, h16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mma16<f16>(h16x8 a, h16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <typename T> struct Mfma;
template <> struct Mfma<h16> {
  using frag = h16x8;
  static constexpr int K = 16;   // contraction depth of one MFMA
  static constexpr int KL = 8;   // k values per lane
};
template <> struct Mfma<float> {
  using frag = float;
  static constexpr int K = 2;
  static constexpr int KL = 1;
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row index (within a 32-row C tile) of element v held by lane-half `half`.
__device__ __forceinline__ int c_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

__device__ __forceinline__ h16x8 as_h16x8(uint4 u) { return __builtin_bit_cast(h16x8, u); }

// Element conversions of the simple kernels (cast, preprocess, layout), whose tensors
// are typed by their element type: float, h16 (bf16) or f16.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(h16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ h16 from_f32<h16>(float x) { return (h16)x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }

// Payload conversions of the MFMA kernels (see h16 above).
template <typename E> __device__ __forceinline__ float val(h16 x);
template <> __device__ __forceinline__ float val<h16>(h16 x) { return (float)x; }
template <> __device__ __forceinline__ float val<f16>(h16 x) {
  return (float)__builtin_bit_cast(f16, x);
}
template <typename E> __device__ __forceinline__ h16 rnd(float x);
template <> __device__ __forceinline__ h16 rnd<h16>(float x) { return (h16)x; }
template <> __device__ __forceinline__ h16 rnd<f16>(float x) {
  return __builtin_bit_cast(h16, (f16)x);
}

// Pack eight fp32 values into an E fragment (round to nearest even).
template <typename E> __device__ __forceinline__ h16x8 pack8(const float *x) {
  if constexpr (sizeof(E) == 2 && !__is_same(E, h16)) {
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (f16)x[i];
    return __builtin_bit_cast(h16x8, r);
  } else {
    h16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (h16)x[i];
    return r;
  }
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// max / sum of x over the lane pair (l, l ^ 32) that shares a C-tile column, through
// v_permlane32_swap (a VALU exchange of the two wave halves, no LDS round trip): of
// the two results, lanes 0-31 hold (own, partner) and lanes 32-63 (partner, own).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// The GQA head table of one kv head held in registers: lane l keeps the q-head of member
// l (t0) and of member l + 64 (t1, only when G > 64).  at(j) returns member j's q-head
// for a per-lane j < G through ds_bpermute (a cross-lane read, no LDS allocation); every
// lane of the wave must be active.
struct HeadMap {
  int t0 = 0, t1 = 0;
  __device__ __forceinline__ void init(const int32_t *qhead, int g, int G, int lane) {
    t0 = lane < G ? qhead[g * G + lane] : 0;
    t1 = lane + 64 < G ? qhead[g * G + 64 + lane] : 0;
  }
  __device__ __forceinline__ int at(int j, int G) const {
    const int a = __builtin_amdgcn_ds_bpermute((j & 63) << 2, t0);
    if (G <= 64) return a;
    const int b = __builtin_amdgcn_ds_bpermute((j & 63) << 2, t1);
    return j >= 64 ? b : a;
  }
  // Member j's q-head for a wave-uniform j < min(G, 64).
  __device__ __forceinline__ int at_uniform(int j) const {
    return __builtin_amdgcn_readlane(t0, __builtin_amdgcn_readfirstlane(j));
  }
};

// q-head of member j of kv head g: the table's entry, or g * G + j for the contiguous map.
__device__ __forceinline__ int q_head(const int32_t *qhead, int g, int G, int j) {
  return qhead ? qhead[g * G + j] : g * G + j;
}

// Compensated (Kahan) add of a partial tile sum into a running fp32 accumulator.
// Used on the fp32 path, whose gradients are summed over thousands of terms and
// checked at 1e-5 absolute.
__device__ __forceinline__ void kahan_add(f32x16 &sum, f32x16 &comp, const f32x16 &x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float y = x[i] - comp[i];
    float t = sum[i] + y;
    comp[i] = (t - sum[i]) - y;
    sum[i] = t;
  }
}

// Exponent domain of the fp32 kernels' softmax.  The 16-bit kernels run in base 2 with
// the hardware exp2 (logits pre-multiplied by scale*log2(e)); the fp32 path, whose
// results are checked at 1e-5, runs in base e with the accurate expf/logf so that
// neither the logits nor the stored natural-log LSE pass through a rounded log2(e)
// factor.
template <typename T> struct Softmax;
template <> struct Softmax<float> {
  __device__ static float factor(float scale) { return scale; }
  __device__ static float lse_in(float lse) { return lse; }
  __device__ static float ex(float x) { return expf(x); }
  __device__ static float lse_out(float m, float l) { return m + logf(l); }
};

}  // namespace dkv
