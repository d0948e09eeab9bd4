// dkv_fwd.hip -- forward kernels: online softmax over a shared-prompt KV region and a
// per-sequence KV region in one pass ("DualKV", arXiv 2605.15422, §3.1).  h16 at head
// dims 64 / 96 / 128 runs fwd_h16_kernel (dkv_fwd_bf16.h), head dims 192 / 256 / 512
// the kernels of dkv_wide.hip; this file holds the fp32 kernel and the dispatch.
//
// fp32 kernel: one workgroup (4 waves) owns 128 query rows = bm_tok tokens x G q-heads
// of one kv head (grouped-query attention, §3.1 last paragraph), so every K/V tile
// staged in LDS feeds all G heads.  It walks
//   1. the context tiles of K_P/V_P (keys at logical positions 0..P-1), then
//   2. its own sequence's tiles (logical positions P + r'),
// carrying the running max m, sum l and output o across the switch, so the result
// equals attention over [K_P; K_Ri] stored contiguously (eq. (4)).  Keys are masked
// by logical position (causal shifted by P, optional left window) and by the end of
// each region; tiles that need no mask skip the per-element test.  With P = 0 and
// one region it is plain varlen causal attention: Call 1 (eq. (3)) and the N-copy
// packing (eq. (2)).
//
// Per 64-key tile each wave computes S^T = K Q^T (keys x its 32 query rows) with fp32
// MFMA (v_mfma_f32_32x32x2_f32) and Q held in registers, updates the softmax with one
// lane owning one query row (two lane-halves each hold half the keys; only the max
// crosses halves per tile), then O^T += V^T P^T with P^T taken straight from the S^T
// accumulator, one key per product.  Base-e softmax with accurate expf / logf: the fp32
// path is checked at 1e-5 absolute.
#include "dkv_device.h"
#include "dkv_launch.h"
#include "dkv_tiles.h"
#include "dkv_fwd_bf16.h"

namespace dkv {

template <int HD>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(FwdArgs a) {
  using T = float;
  constexpr int BN = kFwdBN;
  using TC = TileCfg<T, HD, BN>;
  using M = Mfma<T>;
  constexpr int NKC = HD / M::K;   // MFMA steps over the head dim
  constexpr int NDB = HD / 32;     // 32-wide blocks of the output head dim
  constexpr int NKB = BN / 32;     // 32-key blocks per tile
  __shared__ __attribute__((aligned(16))) char smem[2 * TC::kRowBytes];
  char *ks = smem;
  char *vs = smem + TC::kRowBytes;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const QItem it = a.items[blockIdx.x];
  const int g = it.g, seq0 = it.seq_start, seqlen = it.seq_len;
  const int t0 = it.tile * a.bm_tok;
  const int nt = min(a.bm_tok, seqlen - t0);

  // This lane's query row (one column of the S^T tile).
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
  const T *qptr = reinterpret_cast<const T *>(a.q) + (long)(seq0 + t0 + tok) * qld + (long)h * HD;
  typename M::frag qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) qf[kc] = qptr[kc * 2 + half];

  using SM = Softmax<T>;
  const float sf = SM::factor(a.scale);
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  // Key tile ranges of the two regions for this tile of queries.
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

    // S^T = K Q^T for this wave's 32 query rows.
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        s[kb] = mfma(row_frag<T, HD, BN>(ks, kb * 32 + col, kc, half), qf[kc], s[kb]);
    }

    // Scores in the softmax's exponent domain, masked in place.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] *= sf;

    const bool need_mask = (nrows < BN) || (kpos0 + BN - 1 > qmin) ||
                           (wl >= 0 && kpos0 < qmax - wl);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int kk = kb * 32 + c_row(v, half);
          int kp = kpos0 + kk;
          bool vis = (kk < nrows) && (kp <= qpos) && (wl < 0 || kp >= qpos - wl);
          if (!vis) s[kb][v] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = SM::ex(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = SM::ex(s[kb][v] - m_use);
        s[kb][v] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;

    // O^T += V^T P^T, one key per product.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          acc[db] = mfma(row_elem<HD, BN>(vs, kb * 32 + c_row(v, half), db * 32 + col),
                         s[kb][v], acc[db]);
  }

  const float l = l_run + wave_xor32(l_run);
  const float inv = 1.f / l;
  if (row_valid) {
    T *optr = reinterpret_cast<T *>(a.o) + (long)(seq0 + t0 + tok) * qld + (long)h * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int dim = db * 32 + 8 * i + 4 * half;
        float4 w = make_float4(acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv,
                               acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv);
        *reinterpret_cast<float4 *>(optr + dim) = w;
      }
    if (half == 0)
      a.lse[(long)h * a.lse_ld + seq0 + t0 + tok] = SM::lse_out(m_run, l);
  }
}

template <int HD>
static hipError_t launch_fwd_f32(const FwdArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((fwd_f32_kernel<HD>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E, int HD, int HDP = HD>
static hipError_t fwd_h16(const FwdArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((fwd_h16_kernel<E, HD, kFwdBN, 2, HDP>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Head dim 192 at 32-key tiles of 256-wide rows: 64 KB of LDS and 246 registers, so two
// workgroups per CU and two waves per SIMD.
template <typename E>
static hipError_t fwd_h16_192(const FwdArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((fwd_h16_kernel<E, 192, 32, 2, 256>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int hd, const FwdArgs &a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == 0 || dtype == 2) {   // bf16, fp16
    const bool f = dtype == 2;
    switch (hd) {
      case 64: return f ? fwd_h16<f16, 64>(a, n, s) : fwd_h16<h16, 64>(a, n, s);
      case 96: return f ? fwd_h16<f16, 96, 128>(a, n, s) : fwd_h16<h16, 96, 128>(a, n, s);
      case 128: return f ? fwd_h16<f16, 128>(a, n, s) : fwd_h16<h16, 128>(a, n, s);
      case 192: return f ? fwd_h16_192<f16>(a, n, s) : fwd_h16_192<h16>(a, n, s);
      case 256:
      case 512: return launch_fwd_wide(dtype, hd, a, n, s);
      default: break;
    }
  } else {
    if (hd == 64) return launch_fwd_f32<64>(a, n, s);
    if (hd == 96) return launch_fwd_f32<96>(a, n, s);
    if (hd == 128) return launch_fwd_f32<128>(a, n, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dkv
