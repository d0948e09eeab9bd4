// dkv_bwd.hip -- backward kernels ("DualKV", arXiv 2605.15422, §3.2 and App. A.4).
//
// For each visible (query row t, key j) pair of one q-head:
//   p  = exp(scale * <q_t, k_j> - lse_t)        (recomputed from the forward's LSE)
//   dP = <dO_t, v_j>,   dS = p * (dP - D_t),    D_t = <dO_t, O_t>
//   dQ_t += scale * dS * k_j,   dK_j += scale * dS * q_t,   dV_j += p * dO_t
// Kernels (each h16 kernel has an fp32 counterpart for the 1e-5 parity workload;
// head dims 192, 256 and 512 are in dkv_wide.hip):
//   bwd_pre   D = rowsum(dO * O) in fp32 (the auxiliary preprocessing launch), stored
//             negated, and the LSE in units of the raw dot product, -LSE / scale;
//             the fp32 path only: the h16 dQ kernel forms both for its rows
//   bwd_dq    query-parallel: a workgroup keeps 128 query rows in registers and
//             walks the shared-prompt key tiles, then its own sequence's tiles,
//             exactly like the forward; dQ is written once, no atomics.
//   bwd_dkdv  key-parallel: a workgroup owns 128 keys (V and the dK, dV accumulators
//             in registers, K in LDS) and walks the query rows that see them.
//             Response keys are written directly; shared-prompt keys are visited
//             once per chunk of sequences and their partial dK_P, dV_P summed into
//             the caller's fp32 accumulator with atomic adds (§3.2 "fp32 atomic
//             accumulation", eq. (6)), or stored into the chunk's slice (split mode)
//             for split_reduce to add in slice order.
//   cast      the accumulator is rounded to the tensor dtype once (§3.2 Stage 2).
// In the h16 kernels, transposed operands (contractions over query rows or key rows)
// are read from the same row-layout LDS tiles with the gfx950 transpose read.
#include <type_traits>

#include "dkv_device.h"
#include "dkv_launch.h"
#include "dkv_tiles.h"

namespace dkv {

// ------------------------------------------------------------------ bwd_pre --

// Threads per (token, head) row of the preprocess: one per 16-byte chunk, the group
// padded to a power of two (24 chunks at head dim 96 -> 32 lanes) so that a row's lanes
// are aligned inside the wave and the shuffle reduction stays within them.
template <typename T, int HD> struct PreCfg {
  static constexpr int E = 16 / sizeof(T);     // elements per 16-byte chunk
  static constexpr int TPR = HD / E;           // chunks per row
  static constexpr int TPRP = TPR <= 8 ? 8 : TPR <= 16 ? 16 : TPR <= 32 ? 32 : 64;
  static_assert(TPR <= 64, "a row's chunks fit one wave");
};

template <typename T, int HD>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T *o, const T *dout, const float *lse,
                                                      float *Dneg, float *lsn, long T_tok, int Hq,
                                                      float inv_scale) {
  using C = PreCfg<T, HD>;
  constexpr int E = C::E;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / C::TPRP;            // token-major: row = t * Hq + h
  const int ch = gid % C::TPRP;
  float acc = 0.f;
  if (row < T_tok * Hq && ch < C::TPR) {
    uint4 a = *reinterpret_cast<const uint4 *>(o + row * HD + ch * E);
    uint4 b = *reinterpret_cast<const uint4 *>(dout + row * HD + ch * E);
    const T *x = reinterpret_cast<const T *>(&a);
    const T *y = reinterpret_cast<const T *>(&b);
#pragma unroll
    for (int e = 0; e < E; ++e) acc += to_f32(x[e]) * to_f32(y[e]);
  }
#pragma unroll
  for (int off = C::TPRP / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < T_tok * Hq && ch == 0) {
    long t = row / Hq;
    int h = row - t * Hq;
    Dneg[(long)h * T_tok + t] = -acc;
    lsn[(long)h * T_tok + t] = -lse[(long)h * T_tok + t] * inv_scale;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, long n) {
  long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    *reinterpret_cast<float4 *>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (; i < n; ++i) p[i] = 0.f;
  }
}

// Fixed-order sum of the split mode's slices into the accumulator: each element is
// added slice by slice, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void split_reduce_kernel(float *acc, const float *slices,
                                                           int n_slices, long stride, long n) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    float4 v = *reinterpret_cast<const float4 *>(acc + i);
    for (int c = 0; c < n_slices; ++c) {
      const float4 x = *reinterpret_cast<const float4 *>(slices + c * stride + i);
      v.x += x.x;
      v.y += x.y;
      v.z += x.z;
      v.w += x.w;
    }
    *reinterpret_cast<float4 *>(acc + i) = v;
  } else {
    for (long j = i; j < n; ++j) {
      float v = acc[j];
      for (int c = 0; c < n_slices; ++c) v += slices[c * stride + j];
      acc[j] = v;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void cast_kernel(const float *src, T *dst, long n) {
  long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    float4 v = *reinterpret_cast<const float4 *>(src + i);
    dst[i] = from_f32<T>(v.x);
    dst[i + 1] = from_f32<T>(v.y);
    dst[i + 2] = from_f32<T>(v.z);
    dst[i + 3] = from_f32<T>(v.w);
  } else {
    for (; i < n; ++i) dst[i] = from_f32<T>(src[i]);
  }
}

// ------------------------------------------------------------------- bwd_dq --

// fp32 dQ kernel: the query-parallel structure of the h16 one with fp32 MFMA, base-e
// softmax and compensated (Kahan) accumulation, one key per product.
template <int HD>
__global__ __launch_bounds__(256, 1) void bwd_dq_f32_kernel(BwdQArgs a) {
  using T = float;
  constexpr int BN = kFwdBN;
  using TC = TileCfg<T, HD, BN>;
  using M = Mfma<T>;
  constexpr int NKC = HD / M::K;
  constexpr int NDB = HD / 32;
  constexpr int NKB = BN / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * TC::kRowBytes];
  char *ks = smem;
  char *vs = smem + TC::kRowBytes;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const QItem it = a.items[blockIdx.x];
  const int g = it.g, seq0 = it.seq_start, seqlen = it.seq_len;
  const int t0 = it.tile * a.bm_tok;
  const int nt = min(a.bm_tok, seqlen - t0);
  const int qr = wave * 32 + col;
  int tok = qr / a.G;
  const int hj = qr - tok * a.G;
  const bool row_valid = tok < nt;
  if (!row_valid) tok = nt - 1;
  const int h = q_head(a.qhead, g, a.G, hj);
  const int P = it.ctx_len, wl = a.window_left;
  const int qpos = P + t0 + tok;
  const int qmin = P + t0, qmax = P + t0 + nt - 1;
  const long qld = (long)a.Hq * HD;
  const long kld = (long)a.Hkv * HD;
  const long qrow = (long)(seq0 + t0 + tok);

  const T *qptr = reinterpret_cast<const T *>(a.q) + qrow * qld + (long)h * HD;
  const T *dptr = reinterpret_cast<const T *>(a.dout) + qrow * qld + (long)h * HD;
  typename M::frag qf[NKC], df[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    qf[kc] = qptr[kc * 2 + half];
    df[kc] = dptr[kc * 2 + half];
  }
  using SM = Softmax<T>;
  const float sf = SM::factor(a.scale);
  const float lse2 = SM::lse_in(a.lse[(long)h * a.lse_ld + qrow]);
  const float Dq = -a.Dneg[(long)h * a.lse_ld + qrow];

  f32x16 acc[NDB], comp[NDB];   // sums and their Kahan compensation terms
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    acc[db] = zero16();
    comp[db] = zero16();
  }

  KeyTiles<BN> kt;
  kt.init(P, wl, t0, nt);
  const int n_tiles = kt.n;

  const T *kc_base = reinterpret_cast<const T *>(a.k_ctx) + (long)it.ctx_start * kld + (long)g * HD;
  const T *vc_base = reinterpret_cast<const T *>(a.v_ctx) + (long)it.ctx_start * kld + (long)g * HD;
  const T *ko_base = reinterpret_cast<const T *>(a.k_own) + (long)seq0 * kld + (long)g * HD;
  const T *vo_base = reinterpret_cast<const T *>(a.v_own) + (long)seq0 * kld + (long)g * HD;

  RowRegs<T, HD, BN> kregs, vregs;
  auto issue = [&](int i) {
    if (kt.in_ctx(i)) {
      const int s = kt.ctx_start(i);
      kregs.load(kc_base + (long)s * kld, kld, P - s, tid);
      vregs.load(vc_base + (long)s * kld, kld, P - s, tid);
    } else {
      const int s = kt.own_start(i);
      kregs.load(ko_base + (long)s * kld, kld, seqlen - s, tid);
      vregs.load(vo_base + (long)s * kld, kld, seqlen - s, tid);
    }
  };
  if (n_tiles > 0) issue(0);

  for (int i = 0; i < n_tiles; ++i) {
    int nrows, kpos0;
    kt.at(i, P, seqlen, nrows, kpos0);
    __syncthreads();
    kregs.store(ks, tid);
    vregs.store(vs, tid);
    __syncthreads();
    if (i + 1 < n_tiles) issue(i + 1);

    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = zero16();
      dp[kb] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        s[kb] = mfma(row_frag<T, HD, BN>(ks, kb * 32 + col, kc, half), qf[kc], s[kb]);
        dp[kb] = mfma(row_frag<T, HD, BN>(vs, kb * 32 + col, kc, half), df[kc], dp[kb]);
      }
    }
    const bool need_mask = (nrows < BN) || (kpos0 + BN - 1 > qmin) ||
                           (wl >= 0 && kpos0 < qmax - wl);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = SM::ex(fmaf(s[kb][v], sf, -lse2));
        if (need_mask) {
          int kk = kb * 32 + c_row(v, half);
          int kp = kpos0 + kk;
          bool vis = (kk < nrows) && (kp <= qpos) && (wl < 0 || kp >= qpos - wl);
          if (!vis) p = 0.f;
        }
        s[kb][v] = p * (dp[kb][v] - Dq);   // dS^T
      }

    // dQ^T += K^T dS^T, one key per product.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      f32x16 part = zero16();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          part = mfma(row_elem<HD, BN>(ks, kb * 32 + c_row(v, half), db * 32 + col),
                      s[kb][v], part);
      kahan_add(acc[db], comp[db], part);
    }
  }

  if (row_valid) {
    T *optr = reinterpret_cast<T *>(a.dq) + qrow * qld + (long)h * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int dim = db * 32 + 8 * i + 4 * half;
        float4 w = make_float4(acc[db][4 * i] * a.scale, acc[db][4 * i + 1] * a.scale,
                               acc[db][4 * i + 2] * a.scale, acc[db][4 * i + 3] * a.scale);
        *reinterpret_cast<float4 *>(optr + dim) = w;
      }
  }
}

// h16 dQ kernel with two waves per SIMD: K and V tiles double-buffered in LDS
// through buffer loads (one barrier per 64-key tile), each tile taken as two 32-key
// halves so that Sᵀ, dPᵀ and dSᵀ of one half are live at a time.
// HDP >= HD: the width of the staged rows (as in the forward).
template <typename E, int HD, int HDP = HD>
__global__ __launch_bounds__(256, 2) void bwd_dq_h16_kernel(BwdQArgs a) {
  constexpr int BN = kFwdBN;
  constexpr int TILE = BN * HDP * 2;
  constexpr int NKC = HD / 16;
  constexpr int NDB = HD / 32;
  __shared__ __attribute__((aligned(16))) char smem[2][2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const QItem it = a.items[blockIdx.x];
  const int g = it.g, seq0 = it.seq_start, seqlen = it.seq_len;
  const int t0 = it.tile * a.bm_tok;
  const int nt = min(a.bm_tok, seqlen - t0);
  const int qr = wave * 32 + col;
  int tok = qr / a.G;
  const int hj = qr - tok * a.G;
  const bool row_valid = tok < nt;
  if (!row_valid) tok = nt - 1;
  const int h = q_head(a.qhead, g, a.G, hj);
  const int P = it.ctx_len, wl = a.window_left;
  const int qpos = P + t0 + tok;
  const int qmin = P + t0, qmax = P + t0 + nt - 1;
  const long qld = (long)a.Hq * HD;
  const long kld = (long)a.Hkv * HD;
  const long qrow = (long)(seq0 + t0 + tok);

  const h16 *qptr = reinterpret_cast<const h16 *>(a.q) + qrow * qld + (long)h * HD;
  const h16 *dptr = reinterpret_cast<const h16 *>(a.dout) + qrow * qld + (long)h * HD;
  h16x8 qf[NKC], df[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    qf[kc] = as_h16x8(*reinterpret_cast<const uint4 *>(qptr + kc * 16 + half * 8));
    df[kc] = as_h16x8(*reinterpret_cast<const uint4 *>(dptr + kc * 16 + half * 8));
  }
  const float sf = a.scale * kLog2e;
  const float lse = a.lse[(long)h * a.lse_ld + qrow];
  const float lse2 = lse * kLog2e;
  // D = rowsum(dO ∘ O) of this lane's row (the preprocess step of the backward, done
  // here): the two lanes of a row each hold half of it, in the dO fragments' layout.
  const h16 *optr = reinterpret_cast<const h16 *>(a.o) + qrow * qld + (long)h * HD;
  float Dq = 0.f;
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const h16x8 o8 = as_h16x8(*reinterpret_cast<const uint4 *>(optr + kc * 16 + half * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) Dq += val<E>(o8[e]) * val<E>(df[kc][e]);
  }
  Dq = pair_sum(Dq);
  // The dK/dV kernel, which runs next, reads -D and -LSE / scale of every row.
  if (row_valid && half == 0) {
    a.Dneg_out[(long)h * a.lse_ld + qrow] = -Dq;
    a.lsn_out[(long)h * a.lse_ld + qrow] = -lse * (1.0f / a.scale);
  }
  // dP accumulators start from -D (this lane's row): the products end as dP - D.
  f32x16 negd;
#pragma unroll
  for (int v = 0; v < 16; ++v) negd[v] = -Dq;

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  KeyTiles<BN> kt;
  kt.init(P, wl, t0, nt);
  const int n_tiles = kt.n;

  const h16 *kc_base = reinterpret_cast<const h16 *>(a.k_ctx) + (long)it.ctx_start * kld + (long)g * HD;
  const h16 *vc_base = reinterpret_cast<const h16 *>(a.v_ctx) + (long)it.ctx_start * kld + (long)g * HD;
  const h16 *ko_base = reinterpret_cast<const h16 *>(a.k_own) + (long)seq0 * kld + (long)g * HD;
  const h16 *vo_base = reinterpret_cast<const h16 *>(a.v_own) + (long)seq0 * kld + (long)g * HD;
  const int kld_b = (int)(kld * 2);
  DmaRows<HDP, BN, HD> dma;
  dma.init(wave, lane, kld_b);
  auto issue = [&](int i) {   // tile i -> stage i % 2
    char *st = smem[i & 1];
    if (kt.in_ctx(i)) {
      const int s = kt.ctx_start(i);
      dma.load(st, kc_base + (long)s * kld, kld_b, P - s, wave);
      dma.load(st + TILE, vc_base + (long)s * kld, kld_b, P - s, wave);
    } else {
      const int s = kt.own_start(i);
      dma.load(st, ko_base + (long)s * kld, kld_b, seqlen - s, wave);
      dma.load(st + TILE, vo_base + (long)s * kld, kld_b, seqlen - s, wave);
    }
  };
  if (n_tiles > 0) issue(0);

  for (int i = 0; i < n_tiles; ++i) {
    int nrows, kpos0;
    kt.at(i, P, seqlen, nrows, kpos0);
    dma_wait();
    __syncthreads();
    if (i + 1 < n_tiles) issue(i + 1);
    const char *ks = smem[i & 1];
    const char *vs = smem[i & 1] + TILE;
    const bool need_mask = (nrows < BN) || (kpos0 + BN - 1 > qmin) ||
                           (wl >= 0 && kpos0 < qmax - wl);

#pragma unroll
    for (int hb = 0; hb < BN / 32; ++hb) {
      f32x16 st = zero16(), dpt = negd;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        st = mma16<E>(sw_frag<HDP>(ks, hb * 32 + col, kc, half), qf[kc], st);
        dpt = mma16<E>(sw_frag<HDP>(vs, hb * 32 + col, kc, half), df[kc], dpt);
      }
      float ds[16];
      // The visibility test is compiled only into the variant for tiles that need it.
      auto grads = [&](auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
        // Visible keys of this lane's row, as offsets r = 8 * (v / 4) + v % 4 from the
        // lane's first key hb * 32 + 4 * half: [lo, hi).
        const int k0 = hb * 32 + 4 * half;
        const int lo = (wl >= 0 ? qpos - wl - kpos0 : -BN) - k0;
        const int hi = min(nrows, qpos - kpos0 + 1) - k0;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p = fast_exp2(fmaf(st[v], sf, -lse2));
          if (MASKED) {
            const int r = 8 * (v >> 2) + (v & 3);
            if (r < lo || r >= hi) p = 0.f;
          }
          ds[v] = p * dpt[v];
        }
      };
      if (need_mask)
        grads(std::true_type{});
      else
        grads(std::false_type{});
      const h16x8 d0 = pack8<E>(ds), d1 = pack8<E>(ds + 8);
      // dQᵀ += Kᵀ dSᵀ.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        acc[db] = mma16<E>(sw_tr_frag<HDP>(ks, hb * 32, db * 32, lane), d0, acc[db]);
        acc[db] = mma16<E>(sw_tr_frag<HDP>(ks, hb * 32 + 16, db * 32, lane), d1, acc[db]);
      }
    }
  }

  if (row_valid) {
    h16 *optr = reinterpret_cast<h16 *>(a.dq) + qrow * qld + (long)h * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int dim = db * 32 + 8 * i + 4 * half;
        h16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = rnd<E>(acc[db][4 * i + e] * a.scale);
        *reinterpret_cast<h16x4 *>(optr + dim) = w;
      }
  }
}

// ----------------------------------------------------------------- bwd_dkdv --

// Query-step rows: 32 flattened (token, head) rows of one kv head's G q-heads (fp32).
template <int HD> struct QStepRegs : RowRegs<float, HD, kBwdBM> {
  using T = float;
  using C = TileCfg<T, HD, kBwdBM>;
  // base: row 0 of the sequence, q-head 0; rows f0 .. f0+31 of the flattened (token,
  // member j of kv head g) index, loaded where flo <= row < fend (else zero).
  __device__ __forceinline__ void load_flat(const T *base, long qld, int G, int g,
                                            const int32_t *qhead, int f0, int flo, int fend,
                                            int tid) {
    constexpr int per_row = HD / 4;   // 16-byte chunks per row
#pragma unroll
    for (int p = 0; p < C::kRowPasses; ++p) {
      int id = p * 256 + tid;
      int row = id / per_row, ch = id % per_row;
      int f = f0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (id < C::kChunks && f >= flo && f < fend) {
        int t = f / G, j = f - t * G;
        v = *reinterpret_cast<const uint4 *>(base + (long)t * qld +
                                             (long)q_head(qhead, g, G, j) * HD + ch * 4);
      }
      this->r[p] = v;
    }
  }
};

// fp32 dK/dV kernel: 128 keys per workgroup with K, V and the sums in registers, query
// rows staged through registers into LDS; fp32 MFMA, base-e softmax and compensated
// (Kahan) accumulation, one query row per product.
template <int HD>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_f32_kernel(BwdKVArgs a) {
  using T = float;
  constexpr int BM = kBwdBM;          // query rows per step
  constexpr int BNW = kBwdBN;         // keys per workgroup (4 waves x 32)
  using TC = TileCfg<T, HD, BM>;
  using M = Mfma<T>;
  constexpr int NKC = HD / M::K;
  constexpr int NDB = HD / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * TC::kRowBytes + 2 * BM * 4];
  char *qs = smem;
  char *dos = smem + TC::kRowBytes;
  float *lse_s = reinterpret_cast<float *>(smem + 2 * TC::kRowBytes);
  float *d_s = lse_s + BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const KVItem it = a.items[blockIdx.x];
  const int g = it.g, G = a.G, P = it.ctx_len, wl = a.window_left;
  const bool ctx = it.region == kRegionCtx;
  const long qld = (long)a.Hq * HD;
  const long kld = (long)a.Hkv * HD;
  const int own0 = ctx ? it.ctx_start : sload_i32(a.cu, it.seq_lo);                  // row of the own sequence
  const int nkeys = ctx ? P - it.key_start : sload_i32(a.cu, it.seq_lo + 1) - own0 - it.key_start;
  const int kbase = ctx ? 0 : P;                               // logical position offset
  const int nk_tile = min(BNW, nkeys);

  // This lane's key (one column of the S tile) and its K, V fragments.
  const int kw0 = 32 * wave;                                   // wave's first key in tile
  const int key = kw0 + col;
  const bool key_valid = key < nkeys;
  using SM = Softmax<T>;
  const float sf = SM::factor(a.scale);
  const T *kp = reinterpret_cast<const T *>(ctx ? a.k_ctx : a.k_own) +
                (long)(own0 + it.key_start + (key_valid ? key : 0)) * kld + (long)g * HD;
  const T *vp = reinterpret_cast<const T *>(ctx ? a.v_ctx : a.v_own) +
                (long)(own0 + it.key_start + (key_valid ? key : 0)) * kld + (long)g * HD;
  typename M::frag kf[NKC], vf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    kf[kc] = key_valid ? kp[kc * 2 + half] : 0.f;
    vf[kc] = key_valid ? vp[kc * 2 + half] : 0.f;
  }
  const bool wave_active = kw0 < nkeys;

  f32x16 dk[NDB], dv[NDB];
  f32x16 ck[NDB], cv[NDB];   // Kahan compensation terms
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
    ck[db] = zero16();
    cv[db] = zero16();
  }

  // Steps of BM flattened rows (RowSteps), walked from the last visible row of the last
  // sequence backward.
  RowSteps<BM> rs;
  rs.init(a.cu, it, nk_tile, P, wl, G, ctx, 0);

  QStepRegs<HD> qregs, dregs;
  float lse_r = INFINITY, d_r = 0.f;
  auto issue = [&]() {
    const int cf = rs.cf, s0 = rs.cs0;
    const int lo = max(cf, rs.cfa), hi = min(cf + BM, rs.cfb);
    const T *qb = reinterpret_cast<const T *>(a.q) + (long)s0 * qld;
    const T *db_ = reinterpret_cast<const T *>(a.dout) + (long)s0 * qld;
    qregs.load_flat(qb, qld, G, g, a.qhead, cf, lo, hi, tid);
    dregs.load_flat(db_, qld, G, g, a.qhead, cf, lo, hi, tid);
    if (tid < BM) {
      int f = cf + tid;
      if (f >= lo && f < hi) {
        int t = f / G, j = f - t * G;
        long idx = (long)q_head(a.qhead, g, G, j) * a.lse_ld + s0 + t;
        lse_r = SM::lse_in(a.lse[idx]);
        d_r = -a.Dneg[idx];
      } else {
        lse_r = INFINITY;
        d_r = 0.f;
      }
    }
  };
  if (!rs.done) issue();

  while (!rs.done) {
    int f0, flo, fend;
    rs.advance(f0, flo, fend);
    __syncthreads();
    qregs.store(qs, tid);
    dregs.store(dos, tid);
    if (tid < BM) {
      lse_s[tid] = lse_r;
      d_s[tid] = d_r;
    }
    __syncthreads();
    if (!rs.done) issue();

    if (wave_active) {
      // S = Q K^T and dP = dO V^T for 32 query rows x this wave's 32 keys.
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        s = mfma(row_frag<T, HD, BM>(qs, col, kc, half), kf[kc], s);
        dp = mfma(row_frag<T, HD, BM>(dos, col, kc, half), vf[kc], dp);
      }
      const int ta = flo / G;
      const int tb = (fend - 1) / G;
      const int qpa = P + ta, qpb = P + tb;
      const int kpa = kbase + it.key_start + kw0;
      const int kpb = kbase + it.key_start + min(kw0 + 32, nkeys) - 1;
      const bool full = (flo == f0) && (f0 + BM <= fend) && (kw0 + 32 <= nkeys) && (kpb <= qpa) &&
                        (wl < 0 || kpa >= qpb - wl);
      const int kpos = kbase + it.key_start + key;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 l4 = *reinterpret_cast<const float4 *>(lse_s + 8 * i + 4 * half);
        float4 d4 = *reinterpret_cast<const float4 *>(d_s + 8 * i + 4 * half);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * i + e;
          float p = SM::ex(fmaf(s[v], sf, -lv[e]));
          if (!full) {
            int f = f0 + c_row(v, half);
            int qp = P + f / G;
            bool vis = (f >= flo) && (f < fend) && key_valid && (kpos <= qp) &&
                       (wl < 0 || kpos >= qp - wl);
            if (!vis) p = 0.f;
          }
          s[v] = p;                          // P
          dp[v] = p * (dp[v] - dv4[e]);      // dS
        }
      }
      // dV += P^T dO and dK += dS^T Q (contractions over the step's query rows).
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x16 pv = zero16(), pk = zero16();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = c_row(v, half);
          pv = mfma(s[v], row_elem<HD, BM>(dos, r, db * 32 + col), pv);
          pk = mfma(dp[v], row_elem<HD, BM>(qs, r, db * 32 + col), pk);
        }
        kahan_add(dv[db], cv[db], pv);
        kahan_add(dk[db], ck[db], pk);
      }
    }
  }

  // Epilogue: lane holds dims db*32 + col of keys kw0 + c_row(v, half).
  if (!wave_active) return;
  const bool to_acc = ctx || a.own_to_acc;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = kw0 + c_row(v, half);
      if (k >= nkeys) continue;
      const long off = (long)(own0 + it.key_start + k) * kld + (long)g * HD + db * 32 + col;
      const float gk = dk[db][v] * a.scale;
      const float gv = dv[db][v];
      if (ctx && a.split_dk) {   // split mode: the chunk's own slice, one writer
        const long so = (long)(it.seq_lo / a.split_chunk) * a.split_stride + off;
        a.split_dk[so] = gk;
        a.split_dv[so] = gv;
      } else if (to_acc) {
        atomicAdd(a.acc_dk + off, gk);
        atomicAdd(a.acc_dv + off, gv);
      } else {
        reinterpret_cast<T *>(a.dk_own)[off] = from_f32<T>(gk);
        reinterpret_cast<T *>(a.dv_own)[off] = from_f32<T>(gv);
      }
    }
}

// h16 dK/dV kernel.  A workgroup owns 128 keys of one region and kv head (32 per
// wave: V fragments and the dK, dV accumulators in registers; the workgroup's K tile
// stays in LDS) and streams the query rows that see them in BM-row steps (BM / 32
// blocks of 32), from the last step backward.  Q, dO, LSE and D of the next step
// stream into LDS by DMA while the current step is computed (double-buffered, one
// barrier per step).  The rows of a step are flattened (token, head-of-group) pairs;
// the rows a lane fetches are fixed within a step, so their token/head split is
// precomputed.  With K read from LDS and 32-row steps a wave fits 256 registers and
// the LDS of two workgroups fits a CU: two waves per SIMD.  MAP: the q-heads of the
// kv head come from the GQA head table (a.qhead) instead of g * G + j.
// HDP >= HD: the width of the staged rows (as in the forward).
template <typename E, int HD, int BM, int WPE, bool MAP, int HDP = HD>
__global__ __launch_bounds__(256, WPE) void bwd_dkdv_h16_kernel(BwdKVArgs a) {
  constexpr int BNW = kBwdBN;
  constexpr int TILE = BM * HDP * 2;
  constexpr int NKC = HD / 16;
  constexpr int NDB = HD / 32;
  constexpr int CPR = HDP / 8;                    // 16-byte chunks per staged row
  constexpr int KPW = TILE / 1024 / 4;            // DMA instructions per wave per tile
  constexpr int STAGE = 2 * TILE + 2 * 64 * 4;
  constexpr int KTILE = BNW * HDP * 2;           // the workgroup's K tile
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE + KTILE];
  char *ktile = smem + 2 * STAGE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const KVItem it = a.items[blockIdx.x];
  const int g = it.g, G = a.G, P = it.ctx_len, wl = a.window_left;
  const bool ctx = it.region == kRegionCtx;
  const long qld = (long)a.Hq * HD;
  const long kld = (long)a.Hkv * HD;
  const int own0 = ctx ? it.ctx_start : sload_i32(a.cu, it.seq_lo);
  const int nkeys = ctx ? P - it.key_start : sload_i32(a.cu, it.seq_lo + 1) - own0 - it.key_start;
  const int kbase = ctx ? 0 : P;
  const int nk_tile = min(BNW, nkeys);

  const int kw0 = 32 * wave;
  const int key = kw0 + col;
  const bool key_valid = key < nkeys;
  const float sf = a.scale * kLog2e;
  const h16 *kp = reinterpret_cast<const h16 *>(ctx ? a.k_ctx : a.k_own) +
                   (long)(own0 + it.key_start + (key_valid ? key : 0)) * kld + (long)g * HD;
  const h16 *vp = reinterpret_cast<const h16 *>(ctx ? a.v_ctx : a.v_own) +
                   (long)(own0 + it.key_start + (key_valid ? key : 0)) * kld + (long)g * HD;
  (void)kp;
  h16x8 vf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    vf[kc] = as_h16x8(key_valid ? *reinterpret_cast<const uint4 *>(vp + kc * 16 + half * 8) : z);
  }
  {   // the workgroup's K tile (rows past the region's end are zero-filled)
    DmaRows<HDP, BNW, HD> kd;
    kd.init(wave, lane, (int)(kld * 2));
    kd.load(ktile,
            reinterpret_cast<const h16 *>(ctx ? a.k_ctx : a.k_own) +
                (long)(own0 + it.key_start) * kld + (long)g * HD,
            (int)(kld * 2), nkeys, wave);
  }
  const bool wave_active = kw0 < nkeys;
  // A block of 32 flattened rows [b0, b0 + 32) inside the step's rows needs no mask when
  // every key of the wave sees every row: b0 >= the first row the wave's last key sees,
  // and b0 + 32 <= the end of the rows its first key sees (window).
  const int wkpa = kbase + it.key_start + kw0;
  const int full_lo = __builtin_amdgcn_readfirstlane(
      kw0 + 32 <= nkeys ? max(0, (wkpa + 31 - P) * G) : 0x7fffffff);
  const int full_hi = __builtin_amdgcn_readfirstlane(
      wl >= 0 ? max(0, (wkpa + wl - P + 1) * G) : 0x7fffffff);
  // Per-lane byte offsets of the fragment chunks of row `col` in a swizzled tile; the
  // wave's K rows kw0 + col share them (kw0 is a multiple of 32, the swizzle reads the
  // row's low four bits).
  int fo[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) fo[kc] = Swz<HDP>::off(col, kc * 2 + half);
  const uint32_t kt_wave = __builtin_amdgcn_readfirstlane(lds_u32(ktile) + kw0 * HDP * 2);
  // Flattened query rows f (token f / G) that see this lane's key: the causal mask
  // (key position <= P + f / G) and the window (key position >= P + f / G - wl) as
  // bounds on f, so the per-element test needs no division.  An invalid key sees none.
  const int kpos = kbase + it.key_start + key;
  const int f_vis_lo = key_valid ? max(0, (kpos - P) * G) : 0x7fffffff;
  const int f_vis_hi = (wl >= 0) ? max(0, (kpos + wl - P + 1) * G) : 0x7fffffff;

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  // Steps of BM flattened rows, walked from the last one backward.
  RowSteps<BM> rs;
  rs.init(a.cu, it, nk_tile, P, wl, G, ctx, 0);

  const int tl = lane / G, jl = lane - tl * G;   // this lane's row of the LSE / D fetch
  // ceil(2^24 / G): r * g_recip >> 24 is r / G exactly for r < 64 and G <= 128 (the
  // rounding error r * (g_recip * G - 2^24) stays below 2^24 / G).
  const uint32_t g_recip = __builtin_amdgcn_readfirstlane(((1u << 24) + (uint32_t)G - 1) / (uint32_t)G);
  const int qld_b = (int)(qld * 2);
  const int head0_b = g * G * HD * 2;
  HeadMap hm;
  if constexpr (MAP) hm.init(a.qhead, g, G, lane);
  // Wave 0 fetches LSE rows, wave 1 D rows.
  const __amdgpu_buffer_rsrc_t r_ld = make_rsrc_u(wave == 0 ? (const void *)a.lsn : (const void *)a.Dneg,
                                                  (uint32_t)((long)a.Hq * a.lse_ld * 4));

  // Fetch the step at the cursor into stage `st`.
  auto issue = [&](char *st) {
    const int s0 = rs.cs0;
    const int len = rs.clen;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc_u(reinterpret_cast<const h16 *>(a.q) + (long)s0 * qld, (uint32_t)len * (uint32_t)qld_b);
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc_u(reinterpret_cast<const h16 *>(a.dout) + (long)s0 * qld, (uint32_t)len * (uint32_t)qld_b);
    const int ft = rs.cf / G, fj = rs.cf - ft * G;
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_u32(st) + wave * 1024);
#pragma unroll
    for (int k = 0; k < KPW; ++k) {
      // the row and chunk this lane fetches into the step's swizzled Q / dO tiles
      const int slot = (k * 4 + wave) * 64 + lane;
      const int r = slot / CPR;
      const int tr_ = (int)(((uint32_t)r * g_recip) >> 24);   // r / G (r < 64, G <= 128)
      int t = ft + tr_, j = fj + (r - tr_ * G);
      if (j >= G) {
        j -= G;
        ++t;
      }
      const int hoff = MAP ? hm.at(j, G) * (HD * 2) : head0_b + j * (HD * 2);
      const int src = (slot % CPR) ^ Swz<HDP>::swz(r);   // source chunk of this slot
      // chunks past a padded row's head dim are out of every buffer's range: zeros
      const int off = (HD == HDP || src < HD / 8) ? t * qld_b + hoff + (src << 4) : 0x7ffffff0;
      dma16(rq, l0 + k * 4096, off);
      dma16(rd, l0 + TILE + k * 4096, off);
    }
    if (wave < 2) {   // LSE (wave 0) and D (wave 1) of the step's rows; lanes >= BM read nothing
      int t = ft + tl, j = fj + jl;
      if (j >= G) {
        j -= G;
        ++t;
      }
      const int hq = MAP ? hm.at(j, G) : g * G + j;
      const int off = lane < BM ? (hq * a.lse_ld + s0 + t) * 4 : 0x7fffffff;
      const uint32_t la = __builtin_amdgcn_readfirstlane(lds_u32(st + 2 * TILE) + wave * 256);
      dma4(r_ld, la, off);
    }
  };

  bool have = !rs.done;
  int f0 = 0, flo = 0, fend = 0;
  if (have) {
    issue(smem);
    rs.advance(f0, flo, fend);
  }

  // One step computed from stage STG (a compile-time stage, so every LDS read of the
  // step takes an immediate offset) while the next step streams into the other.
  auto step = [&](auto stg_c) {
    constexpr int STG = decltype(stg_c)::value;
    dma_wait();
    __syncthreads();
    const bool more = !rs.done;
    int g0 = 0, glo = 0, gend = 0;
    if (more) {
      issue(smem + (STG ^ 1) * STAGE);
      rs.advance(g0, glo, gend);
    }
    const char *qs = smem + STG * STAGE;
    const char *dos = qs + TILE;
    const float *lsn_s = reinterpret_cast<const float *>(qs + 2 * TILE);
    const float *dn_s = lsn_s + 64;

    if (wave_active) {
      // Recomputed each step (opaque to the compiler) so the K addresses below stay one
      // add each instead of eight live registers.
      uint32_t kt = kt_wave;
      asm volatile("" : "+s"(kt));
#pragma unroll
      for (int rb = 0; rb < BM / 32; ++rb) {
        const int b0 = f0 + rb * 32;
        if (b0 + 32 <= flo || b0 >= fend) continue;   // block outside the step's rows
        // The accumulators start at -LSE / scale and -D of their rows, so they end as
        // <q, k> - LSE / scale and dP - D.
        f32x16 st, dpt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 l4 = *reinterpret_cast<const float4 *>(lsn_s + rb * 32 + 8 * i + 4 * half);
          const float4 d4 = *reinterpret_cast<const float4 *>(dn_s + rb * 32 + 8 * i + 4 * half);
          st[4 * i] = l4.x, st[4 * i + 1] = l4.y, st[4 * i + 2] = l4.z, st[4 * i + 3] = l4.w;
          dpt[4 * i] = d4.x, dpt[4 * i + 1] = d4.y, dpt[4 * i + 2] = d4.z, dpt[4 * i + 3] = d4.w;
        }
        // MFMA stretches run at raised wave priority: with two waves per SIMD, the one
        // ready to issue matrix work goes first and the other's softmax fills the gaps.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const char *qrow = qs + rb * 32 * HDP * 2 + fo[kc];
          st = mma16<E>(as_h16x8(*reinterpret_cast<const uint4 *>(qrow)), lds_frag_at(kt + fo[kc]), st);
          dpt = mma16<E>(as_h16x8(*reinterpret_cast<const uint4 *>(qrow + TILE)), vf[kc], dpt);
        }
        // three fragment reads (Q, K, dO) ahead of each pair of products
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int kc = 0; kc < NKC - 2; ++kc) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_s_setprio(0);
        const bool full = b0 >= max(flo, full_lo) && b0 + 32 <= min(fend, full_hi);
        float pv[16], dsv[16];
        // P and dS of the block; the visibility test is compiled only into the masked
        // variant, which runs on the few blocks that straddle a mask edge or a range end.
        auto probs = [&](auto masked_c) {
          constexpr bool MASKED = decltype(masked_c)::value;
          // Rows b0 + c_row(v, half) in [vlo, vhi) are visible: as offsets from this
          // lane's first row, [lo, hi).
          const int lo = max(flo, f_vis_lo) - b0 - 4 * half;
          const int hi = min(fend, f_vis_hi) - b0 - 4 * half;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float p = fast_exp2(st[v] * sf);
            if (MASKED) {
              const int r = 8 * (v >> 2) + (v & 3);
              if (r < lo || r >= hi) p = 0.f;
            }
            pv[v] = p;
            dsv[v] = p * dpt[v];
          }
        };
        if (full)
          probs(std::false_type{});
        else
          probs(std::true_type{});
        const h16x8 p0 = pack8<E>(pv), p1 = pack8<E>(pv + 8);
        const h16x8 s0 = pack8<E>(dsv), s1 = pack8<E>(dsv + 8);
        // dV += Pᵀ dO and dK += dSᵀ Q over the block's 32 rows.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dv[db] = mma16<E>(p0, sw_tr_frag<HDP>(dos, rb * 32, db * 32, lane), dv[db]);
          dv[db] = mma16<E>(p1, sw_tr_frag<HDP>(dos, rb * 32 + 16, db * 32, lane), dv[db]);
          dk[db] = mma16<E>(s0, sw_tr_frag<HDP>(qs, rb * 32, db * 32, lane), dk[db]);
          dk[db] = mma16<E>(s1, sw_tr_frag<HDP>(qs, rb * 32 + 16, db * 32, lane), dk[db]);
        }
        // transposed dO / Q reads three products ahead
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int j = 0; j < 4 * NDB - 3; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    have = more;
    f0 = g0, flo = glo, fend = gend;
  };
  while (have) {
    step(std::integral_constant<int, 0>{});
    if (!have) break;
    step(std::integral_constant<int, 1>{});
  }

  // Epilogue: lane holds dims db*32 + col of keys kw0 + c_row(v, half).
  if (!wave_active) return;
  const bool to_acc = ctx || a.own_to_acc;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = kw0 + c_row(v, half);
      if (k >= nkeys) continue;
      const long off = (long)(own0 + it.key_start + k) * kld + (long)g * HD + db * 32 + col;
      const float gk = dk[db][v] * a.scale;
      const float gv = dv[db][v];
      if (ctx && a.split_dk) {   // split mode: the chunk's own slice, one writer
        const long so = (long)(it.seq_lo / a.split_chunk) * a.split_stride + off;
        a.split_dk[so] = gk;
        a.split_dv[so] = gv;
      } else if (to_acc) {
        atomicAdd(a.acc_dk + off, gk);
        atomicAdd(a.acc_dv + off, gv);
      } else {
        reinterpret_cast<h16 *>(a.dk_own)[off] = rnd<E>(gk);
        reinterpret_cast<h16 *>(a.dv_own)[off] = rnd<E>(gv);
      }
    }
}

// ---------------------------------------------------------------- launchers --

template <typename T, int HD>
static hipError_t pre_t(const void *o, const void *dout, const float *lse, float *Dneg, float *lsn,
                        long T_tok, int Hq, float scale, hipStream_t s) {
  long threads = T_tok * Hq * PreCfg<T, HD>::TPRP;
  long blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((bwd_pre_kernel<T, HD>), dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const T *>(o), reinterpret_cast<const T *>(dout), lse, Dneg,
                     lsn, T_tok, Hq, 1.0f / scale);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(int dtype, int hd, const void *o, const void *dout, const float *lse,
                          float *Dneg, float *lsn, long T, int Hq, float scale, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dtype == 1) {   // fp32 only: the h16 dQ kernels form these terms themselves
    if (hd == 64) return pre_t<float, 64>(o, dout, lse, Dneg, lsn, T, Hq, scale, s);
    if (hd == 96) return pre_t<float, 96>(o, dout, lse, Dneg, lsn, T, Hq, scale, s);
    if (hd == 128) return pre_t<float, 128>(o, dout, lse, Dneg, lsn, T, Hq, scale, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fill_zero(float *p, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long blocks = (n + 1023) / 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_split_reduce(float *acc, const float *slices, int n_slices, long stride,
                               long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long blocks = (n + 1023) / 1024;
  hipLaunchKernelGGL(split_reduce_kernel, dim3(blocks), dim3(256), 0, s, acc, slices, n_slices,
                     stride, n);
  return hipGetLastError();
}

hipError_t launch_cast(int dtype, const float *src, void *dst, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long blocks = (n + 1023) / 1024;
  if (dtype == 2)
    hipLaunchKernelGGL(cast_kernel<f16>, dim3(blocks), dim3(256), 0, s, src,
                       reinterpret_cast<f16 *>(dst), n);
  else if (dtype == 0)
    hipLaunchKernelGGL(cast_kernel<h16>, dim3(blocks), dim3(256), 0, s, src,
                       reinterpret_cast<h16 *>(dst), n);
  else
    hipLaunchKernelGGL(cast_kernel<float>, dim3(blocks), dim3(256), 0, s, src,
                       reinterpret_cast<float *>(dst), n);
  return hipGetLastError();
}

template <int HD>
static hipError_t dq_f32(const BwdQArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dq_f32_kernel<HD>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E, int HD, int HDP = HD>
static hipError_t dq_h16(const BwdQArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dq_h16_kernel<E, HD, HDP>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(int dtype, int hd, const BwdQArgs &a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == 0 || dtype == 2) {   // bf16, fp16
    const bool f = dtype == 2;
    switch (hd) {
      case 64: return f ? dq_h16<f16, 64>(a, n, s) : dq_h16<h16, 64>(a, n, s);
      case 96: return f ? dq_h16<f16, 96, 128>(a, n, s) : dq_h16<h16, 96, 128>(a, n, s);
      case 128: return f ? dq_h16<f16, 128>(a, n, s) : dq_h16<h16, 128>(a, n, s);
      case 192:
      case 256:
      case 512: return launch_bwd_dq_wide(dtype, hd, a, n, s);
      default: break;
    }
  } else {
    if (hd == 64) return dq_f32<64>(a, n, s);
    if (hd == 96) return dq_f32<96>(a, n, s);
    if (hd == 128) return dq_f32<128>(a, n, s);
  }
  return hipErrorInvalidValue;
}

template <int HD>
static hipError_t dkdv_f32(const BwdKVArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<HD>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E, int HD, int HDP = HD>
static hipError_t dkdv_h16(const BwdKVArgs &a, int n, hipStream_t s) {
  if (a.qhead)
    hipLaunchKernelGGL((bwd_dkdv_h16_kernel<E, HD, 32, 2, true, HDP>), dim3(n), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_h16_kernel<E, HD, 32, 2, false, HDP>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(int dtype, int hd, const BwdKVArgs &a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == 0 || dtype == 2) {   // bf16, fp16
    const bool f = dtype == 2;
    switch (hd) {
      case 64: return f ? dkdv_h16<f16, 64>(a, n, s) : dkdv_h16<h16, 64>(a, n, s);
      case 96: return f ? dkdv_h16<f16, 96, 128>(a, n, s) : dkdv_h16<h16, 96, 128>(a, n, s);
      case 128: return f ? dkdv_h16<f16, 128>(a, n, s) : dkdv_h16<h16, 128>(a, n, s);
      case 192:
      case 256:
      case 512: return launch_bwd_dkdv_wide(dtype, hd, a, n, s);
      default: break;
    }
  } else {
    if (hd == 64) return dkdv_f32<64>(a, n, s);
    if (hd == 96) return dkdv_f32<96>(a, n, s);
    if (hd == 128) return dkdv_f32<128>(a, n, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dkv
