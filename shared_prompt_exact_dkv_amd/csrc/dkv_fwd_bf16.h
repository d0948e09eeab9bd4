// dkv_fwd_bf16.h -- the h16 forward kernel template ("DualKV", arXiv 2605.15422,
// §3.1): one online softmax over the shared-prompt KV region then the sequence's own
// region.  Instantiated in dkv_fwd.hip for head dims 64, 96 and 128 (64-key tiles) and
// 192 (32-key tiles of 256-wide rows); head dims 256 and 512 have their own kernels in
// dkv_wide.hip.
#pragma once

#include "dkv_device.h"
#include "dkv_launch.h"
#include "dkv_tiles.h"

namespace dkv {

// ------------------------------------------------------------- h16 kernel --
//
// The h16 path for head dims 64 to 192: BN-key tiles (64; 32 at head dim 192, where Q
// and O take 144 registers) at two waves per SIMD (WPE = 2, <= 256 registers).
//   - K and V tiles are dense swizzled tiles filled by LDS DMA, double-buffered with
//     one barrier per tile: the next tile streams in while the current one is
//     computed.
//   - Vᵀ (the A operand of Oᵀ += Vᵀ Pᵀ) comes straight from the row-layout tile
//     through the gfx950 transpose read, in the key order of the Sᵀ accumulator.
//   - The softmax scale is folded into the exponent (one FMA per score), and the
//     output is rescaled only when a row's running maximum grows by more than
//     kSlack (log2 units): between rescales the probabilities are exp2(t - m) with
//     m at most kSlack below the true running maximum, i.e. bounded by 2^kSlack,
//     and O / l and LSE = m + log2(l) are unchanged in exact arithmetic.
//   - HDP >= HD is the width of the staged rows (a power of two; head dim 96 is staged
//     in 128-wide rows whose last chunks read as zeros and are never used).
template <typename E, int HD, int BN, int WPE, int HDP = HD>
__global__ __launch_bounds__(256, WPE) void fwd_h16_kernel(FwdArgs a) {
  constexpr int TILE = BN * HDP * 2;    // dense swizzled tile
  constexpr int NKC = HD / 16;     // MFMA steps over the head dim
  constexpr int NDB = HD / 32;     // 32-wide blocks of the output head dim
  constexpr int NKB = BN / 32;     // 32-key blocks per tile
  constexpr float kSlack = 8.f;
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
  if (!row_valid) tok = nt - 1;   // computes a duplicate of a valid row, never stored
  const int h = q_head(a.qhead, g, a.G, hj);
  const int P = it.ctx_len, wl = a.window_left;
  const int qpos = P + t0 + tok;
  const int qmin = P + t0, qmax = P + t0 + nt - 1;

  const long qld = (long)a.Hq * HD;
  const long kld = (long)a.Hkv * HD;
  const h16 *qptr = reinterpret_cast<const h16 *>(a.q) + (long)(seq0 + t0 + tok) * qld + (long)h * HD;
  h16x8 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    qf[kc] = as_h16x8(*reinterpret_cast<const uint4 *>(qptr + kc * 16 + half * 8));

  const float sf = a.scale * kLog2e;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

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
    // Tile i has landed in stage i % 2 and every wave is done with tile i - 1, whose
    // stage receives tile i + 1 while tile i is computed.
    dma_wait();
    __syncthreads();
    if (i + 1 < n_tiles) issue(i + 1);
    const char *ks = smem[i & 1];
    const char *vs = smem[i & 1] + TILE;

    // Sᵀ = K Qᵀ for this wave's 32 query rows (raw scores).
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mma16<E>(sw_frag<HDP>(ks, kb * 32 + col, kc, half), qf[kc], s[kb]);
    }
    // K fragment reads four products ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int j = 0; j < NKC * NKB - 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    const bool need_mask = (nrows < BN) || (kpos0 + BN - 1 > qmin) ||
                           (wl >= 0 && kpos0 < qmax - wl);
    if (need_mask) {
      // Visible keys of this lane's row as tile offsets [lo, hi): inside the tile,
      // causal, and inside the window; compared per element without branches.
      const int lo = (wl >= 0 ? qpos - wl - kpos0 : -BN) - 4 * half;
      const int hi = min(nrows, qpos - kpos0 + 1) - 4 * half;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = kb * 32 + 8 * (v >> 2) + (v & 3);   // kb * 32 + c_row(v, half) - 4 half
          s[kb][v] = (r >= lo) & (r < hi) ? s[kb][v] : -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = pair_max(mx) * sf;
    const bool grow = mx > m_run + kSlack;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
      if (grow) m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f;
    h16x8 pf[2 * NKB];
#pragma unroll
    for (int u = 0; u < 2 * NKB; ++u) {
      float t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        t[e] = fast_exp2(fmaf(s[u >> 1][8 * (u & 1) + e], sf, -m_use));
        rs += t[e];
      }
      pf[u] = pack8<E>(t);
    }
    l_run += rs;

    // Oᵀ += Vᵀ Pᵀ.
#pragma unroll
    for (int u = 0; u < 2 * NKB; ++u)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        acc[db] = mma16<E>(sw_tr_frag<HDP>(vs, 16 * u, db * 32, lane), pf[u], acc[db]);
      }
  }

  const float l = pair_sum(l_run);
  const float inv = 1.f / l;
  if (row_valid) {
    h16 *optr = reinterpret_cast<h16 *>(a.o) + (long)(seq0 + t0 + tok) * qld + (long)h * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int dim = db * 32 + 8 * i + 4 * half;
        h16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = rnd<E>(acc[db][4 * i + e] * inv);
        *reinterpret_cast<h16x4 *>(optr + dim) = w;
      }
    if (half == 0)
      a.lse[(long)h * a.lse_ld + seq0 + t0 + tok] = (m_run + fast_log2(l)) * kLn2;
  }
}

}  // namespace dkv
