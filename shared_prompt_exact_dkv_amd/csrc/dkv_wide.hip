// dkv_wide.hip -- head dimensions 192, 256 and 512 ("DualKV", arXiv 2605.15422, §3 "Head
// dimensions and sliding-window support": the d = 512 global layers and d = 256
// sliding-window layers of hybrid models; 192 completes the head dims of App. E.1).
//
// A wave's fragments and fp32 accumulators for 32 rows over a wide head dim need up to
// 768 registers, so the kernels share each 32-row (or 32-key) block between waves and
// keep every wave within the architectural VGPRs, two waves per SIMD.  Tiles are staged
// in rows of HDP elements (256 or 512, a power of two); head dim 192 is staged in
// 256-wide rows whose last 64 elements read as zeros (its fragments past the head dim
// are zero, its products there are skipped where whole blocks are padding, and its
// outputs there are never stored), so its backward runs the d = 256 kernels (its
// forward fits the whole-row kernel of dkv_fwd_bf16.h, which is faster there).  Tiles
// are staged by LDS DMA into swizzled dense rows (one 1 KB DMA block holds one 512-wide
// row or two 256-wide rows).
//
//   forward  (both widths) 128 query rows per workgroup of 8 waves; the two waves of
//            a pair share 32 rows and each holds Q and O for one half of the head dim.
//            Each computes the partial scores Sᵀ over its half, the pair adds the two
//            partials through LDS (both in the same order, so both see identical
//            scores), and each accumulates its half of O.  Waves 0-3 run half a tile
//            ahead of waves 4-7, which share their SIMDs.  Double-buffered K / V.
//   dQ, HDP = 512: 64 query rows per workgroup of 8 waves, two groups of four with 32
//            rows each.  In a group, waves 0 / 1 form partial Sᵀ = K Qᵀ over the two
//            halves of the head dim (holding Q), waves 2 / 3 partial dPᵀ = V dOᵀ
//            (holding dO).  After one exchange each wave forms dSᵀ for a quarter of the
//            tile, and after a second every wave reads the whole dSᵀ and accumulates dQ
//            for one quarter of the head dim.
//   dK/dV, HDP = 512: 64 keys per workgroup, the same arrangement: in a group, waves
//            0 / 1 hold K halves and form partial S, waves 2 / 3 hold V halves and form
//            partial dP; P and dS are formed a quarter of the tile per wave and shared,
//            and each wave accumulates dK and dV for one quarter of the head dim.
//            Both double-buffered, three barriers per tile; the exchange area takes
//            the last 32 KB of the 160 KB of LDS.
//   dQ and dK/dV, HDP = 256: pairs of waves, each wave over the whole head dim
//            (bwd_dq_pair_kernel, bwd_dkdv_pair_kernel): 128 rows or keys per
//            workgroup; one wave of a pair forms the scores, the other dP, and the
//            tiles cross through LDS once.  Three stages and a double-buffered exchange
//            area let one barrier per tile hand over both.
#include <type_traits>

#include "dkv_device.h"
#include "dkv_launch.h"
#include "dkv_tiles.h"

namespace dkv {

namespace {

// One 32 x 32 fp32 C tile per wave in the exchange area, as four 1 KB quads: lane l
// keeps elements 4q .. 4q+3 at words 256 q + 4 l .. +3 (16-byte accesses, every bank
// once per quarter wave), and the other waves read the same slots (same C layout).
__device__ __forceinline__ void xch_put(float *area, const f32x16 &x, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<float4 *>(area + q * 256 + lane * 4) =
        make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
}
__device__ __forceinline__ float4 xch_quad(const float *area, int q, int lane) {
  return *reinterpret_cast<const float4 *>(area + q * 256 + lane * 4);
}
// Two floats as an E pair (x in the low half, nearest even), and four such words as an
// 8-element fragment.
template <typename E> __device__ __forceinline__ uint32_t pack2(float x, float y) {
  typedef E e16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, e16x2));
}
__device__ __forceinline__ h16x8 words8(const uint32_t *w) {
  return __builtin_bit_cast(h16x8, make_uint4(w[0], w[1], w[2], w[3]));
}
// Issue order of a run of N products, each fed by R LDS reads: the reads run A
// products ahead (A * R reads first, then a product and the next product's reads, and
// the last A products at the end).
template <int N, int R, int A> __device__ __forceinline__ void reads_ahead() {
  static_assert(A >= 1 && A <= N, "read-ahead depth");
  __builtin_amdgcn_sched_group_barrier(0x100, A * R, 0);
#pragma unroll
  for (int i = 0; i < N - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}

// The key tiles of a query work item (KeyTiles) with the K or V rows they fetch: `v`
// picks the V rows (else K); the wave with index w among the four that fetch a tile
// writes its blocks b % 4 == w (DmaRows).
template <int HD, int HDP, int BN> struct KVTiles : KeyTiles<BN> {
  int P, seqlen, w, kld_b;
  long kld;
  const h16 *c_base, *o_base;
  DmaRows<HDP, BN, HD> dma;
  template <typename Args>
  __device__ __forceinline__ void init(const Args &a, const QItem &it, int t0, int nt, bool v,
                                       int w_, int lane) {
    P = it.ctx_len;
    seqlen = it.seq_len;
    w = w_;
    KeyTiles<BN>::init(P, a.window_left, t0, nt);
    kld = (long)a.Hkv * HD;
    kld_b = (int)(kld * 2);
    c_base = reinterpret_cast<const h16 *>(v ? a.v_ctx : a.k_ctx) + (long)it.ctx_start * kld + (long)it.g * HD;
    o_base = reinterpret_cast<const h16 *>(v ? a.v_own : a.k_own) + (long)it.seq_start * kld + (long)it.g * HD;
    dma.init(w, lane, kld_b);
  }
  __device__ __forceinline__ void at(int i, int &nrows, int &kpos0) const {
    KeyTiles<BN>::at(i, P, seqlen, nrows, kpos0);
  }
  // This wave's share of tile i into the LDS tile at st.
  __device__ __forceinline__ void fetch(char *st, int i) {
    if (this->in_ctx(i)) {
      const int s = this->ctx_start(i);
      dma.load(st, c_base + (long)s * kld, kld_b, P - s, w);
    } else {
      const int s = this->own_start(i);
      dma.load(st, o_base + (long)s * kld, kld_b, seqlen - s, w);
    }
  }
};
}  // namespace

// ------------------------------------------------------------------- forward --

template <typename E, int HD, int HDP>
__global__ __launch_bounds__(512, 1) void fwd_wide_kernel(FwdArgs a) {
  constexpr int BN = 32;
  constexpr int TILE = BN * HDP * 2;     // 32 KB at HDP = 512
  constexpr int NKH = HDP / 2 / 16;      // MFMA k-steps per half head dim
  constexpr int NDH = HDP / 2 / 32;      // 32-wide output blocks per half
  constexpr float kSlack = 8.f;
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE + 8 * 4096];
  float *xch = reinterpret_cast<float *>(smem + 4 * TILE);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int rb = wave >> 1, dh = wave & 1;
  const QItem it = a.items[blockIdx.x];
  const int g = it.g, seq0 = it.seq_start, seqlen = it.seq_len;
  const int t0 = it.tile * a.bm_tok;
  const int nt = min(a.bm_tok, seqlen - t0);
  const int qr = rb * 32 + col;
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
  const int d0 = dh * (HDP / 2);

  const h16 *qptr = reinterpret_cast<const h16 *>(a.q) + (long)(seq0 + t0 + tok) * qld + (long)h * HD + d0;
  h16x8 qf[NKH];
#pragma unroll
  for (int kc = 0; kc < NKH; ++kc)   // dims past the head dim (padded rows) are zero
    qf[kc] = (HD == HDP || d0 + kc * 16 < HD)
                 ? as_h16x8(*reinterpret_cast<const uint4 *>(qptr + kc * 16 + half * 8))
                 : as_h16x8(make_uint4(0, 0, 0, 0));

  const float sf = a.scale * kLog2e;
  f32x16 acc[NDH];
#pragma unroll
  for (int db = 0; db < NDH; ++db) acc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  // Tile i goes to stage i % 2: waves 0-3 fetch its K rows, waves 4-7 its V rows.
  const int dw = wave & 3, isv = wave >> 2;
  KVTiles<HD, HDP, BN> kv;
  kv.init(a, it, t0, nt, isv, dw, lane);
  const int n_tiles = kv.n;
  auto issue = [&](int i) { kv.fetch(smem + (i & 1) * 2 * TILE + isv * TILE, i); };
  SwWide<HDP> sw;
  sw.init(lane);

  // Partial Sᵀ = K Qᵀ of tile i over this wave's half of the head dim, into the
  // wave's exchange slot.
  auto scores = [&](int i) {
    const char *ks = smem + (i & 1) * 2 * TILE;
    f32x16 part = zero16();
#pragma unroll
    for (int kc = 0; kc < NKH; ++kc)
      part = mma16<E>(sw.frag(lds_u32(ks) + dh * HDP, kc), qf[kc], part);
    reads_ahead<NKH, 1, 2>();   // one fragment read per product, two products ahead
    xch_put(xch + wave * 1024, part, lane);
  };
  // Softmax of tile i from the pair's two partials, then Oᵀ += Vᵀ Pᵀ.
  auto accumulate = [&](int i) {
    int nrows, kpos0;
    kv.at(i, nrows, kpos0);
    const char *vs = smem + (i & 1) * 2 * TILE + TILE;
    // Full scores: the pair's partials 0 + 1, both read back a quad at a time (the
    // same bits in both waves of the pair).
    f32x16 s;
    const float *pa = xch + (wave & ~1) * 1024;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x0 = xch_quad(pa, q, lane), x1 = xch_quad(pa + 1024, q, lane);
      s[4 * q] = x0.x + x1.x;
      s[4 * q + 1] = x0.y + x1.y;
      s[4 * q + 2] = x0.z + x1.z;
      s[4 * q + 3] = x0.w + x1.w;
    }

    const bool need_mask = (nrows < BN) || (kpos0 + BN - 1 > qmin) ||
                           (wl >= 0 && kpos0 < qmax - wl);
    if (need_mask) {
      // Visible keys of this lane's row as a range of tile offsets [lo, hi): inside the
      // tile, causal, and inside the window; compared per element without branches.
      const int lo = (wl >= 0 ? qpos - wl - kpos0 : -BN) - 4 * half;
      const int hi = min(nrows, qpos - kpos0 + 1) - 4 * half;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + (v & 3);   // c_row(v, half) - 4 half
        s[v] = ((r >= lo) & (r < hi)) ? s[v] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
    mx = pair_max(mx) * sf;
    const bool grow = mx > m_run + kSlack;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
      if (grow) m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDH; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    uint32_t pw[8];   // P as h16 pairs
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float t0 = fast_exp2(fmaf(s[v], sf, -m_use));
      const float t1 = fast_exp2(fmaf(s[v + 1], sf, -m_use));
      rs += t0;
      rs += t1;
      pw[v / 2] = pack2<E>(t0, t1);
    }
    l_run += rs;
    const h16x8 p0 = words8(pw), p1 = words8(pw + 4);
    // Oᵀ += Vᵀ Pᵀ over this wave's half of the head dim.
#pragma unroll
    for (int db = 0; db < NDH; ++db) {
      acc[db] = mma16<E>(sw.trfrag(lds_u32(vs) + d0 * 2, 0, db), p0, acc[db]);
      acc[db] = mma16<E>(sw.trfrag(lds_u32(vs) + d0 * 2, 16, db), p1, acc[db]);
    }
    reads_ahead<2 * NDH, 2, 2>();   // a transposed fragment (two reads) per product, two ahead
  };

  // Ping-pong: waves 0-3 run half a tile ahead of waves 4-7 (one of each per SIMD), so
  // one group's softmax overlaps the other's products.  Both run the same loop, but
  // waves 4-7 pass one barrier first: in phase 2i waves 0-3 form the scores of tile i
  // while waves 4-7 accumulate tile i - 1, in phase 2i + 1 the reverse.  K of tile i + 1
  // is fetched by waves 0-3 in phase 2i (its stage was last read in phase 2i - 1) and
  // lands before phase 2i + 2; V of tile i + 1 by waves 4-7 in phase 2i + 1 (last read
  // in phase 2i) and lands before phase 2i + 3.  Every wave passes 2 n + 2 barriers.
  const bool lead = wave < 4;
  // The wait is taken on every path, tile or not: it also covers the Q fragments loaded
  // above, so no path reaches the loop with those loads still counted as in flight
  // (the compiler would then wait for them inside the loop, behind the next tile's DMA).
  if (n_tiles > 0) issue(0);
  dma_wait();
  __syncthreads();
  if (!lead) __syncthreads();
  for (int i = 0; i < n_tiles; ++i) {
    sw.opaque();
    if (i + 1 < n_tiles) issue(i + 1);
    scores(i);
    __syncthreads();
    accumulate(i);
    dma_wait();
    __syncthreads();
  }
  if (lead) __syncthreads();

  const float l = pair_sum(l_run);
  const float inv = 1.f / l;
  if (row_valid) {
    h16 *optr = reinterpret_cast<h16 *>(a.o) + (long)(seq0 + t0 + tok) * qld + (long)h * HD + d0;
#pragma unroll
    for (int db = 0; db < NDH; ++db) {
      if (HD != HDP && d0 + db * 32 >= HD) continue;   // padded dims: not stored
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int dim = db * 32 + 8 * i + 4 * half;
        h16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = rnd<E>(acc[db][4 * i + e] * inv);
        *reinterpret_cast<h16x4 *>(optr + dim) = w;
      }
    }
    if (half == 0 && dh == 0)
      a.lse[(long)h * a.lse_ld + seq0 + t0 + tok] = (m_run + fast_log2(l)) * kLn2;
  }
}

// Forward at HDP = 256 (head dim 256; 192 also fits it): 128 query rows per workgroup of 8
// waves, four pairs of 32 rows.  In pair p, wave p (role 0) holds Q of the pair's rows
// over the whole head dim, forms Sᵀ = K Qᵀ, runs the online softmax and accumulates
// the first half of O; wave p + 4 (role 1, on the same SIMD) accumulates the second
// half from the P (packed 16-bit, as the product's operand) and the rows' rescale
// factors that role 0 leaves in LDS.  Three K / V stages and a double-buffered P area
// let one barrier per tile hand over both (each wave waits for its own loads of tile
// i + 1 first; the stage of tile i - 1, finished by every wave at the barrier of tile
// i, takes tile i + 2).  Role 1's products of tile i run beside role 0's scores of
// tile i + 1.
template <typename E, int HD>
__global__ __launch_bounds__(512, 1) void fwd_pair_kernel(FwdArgs a) {
  constexpr int HDP = 256;
  constexpr int BN = 32;
  constexpr int TILE = BN * HDP * 2;     // 16 KB
  constexpr int NKC = HD / 16;           // k-steps over the real head dim
  constexpr int NDH = HDP / 2 / 32;      // 32-wide output blocks per half of the head dim
  constexpr int NST = 3;
  constexpr int PA = 2;                  // fragment reads ahead of the products
  constexpr int XS = 64 * 32 + 64 * 4;   // per pair and buffer: P words, then rescale factors
  constexpr float kSlack = 8.f;
  static_assert(HD == 192 || HD == 256, "head dims staged in 256-wide rows");
  __shared__ __attribute__((aligned(16))) char smem[NST * 2 * TILE + 2 * 4 * XS];
  char *xbase = smem + NST * 2 * TILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int role = wave >> 2, pair = wave & 3;
  const QItem it = a.items[blockIdx.x];
  const int g = it.g, seq0 = it.seq_start, seqlen = it.seq_len;
  const int t0 = it.tile * a.bm_tok;
  const int nt = min(a.bm_tok, seqlen - t0);
  const int qr = pair * 32 + col;
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
  const int d0 = role * (HDP / 2);   // first dim of this wave's half of O

  h16x8 qf[NKC];
  if (role == 0) {
    const h16 *qptr = reinterpret_cast<const h16 *>(a.q) + (long)(seq0 + t0 + tok) * qld + (long)h * HD;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      qf[kc] = as_h16x8(*reinterpret_cast<const uint4 *>(qptr + kc * 16 + half * 8));
  }

  const float sf = a.scale * kLog2e;
  f32x16 acc[NDH];
#pragma unroll
  for (int db = 0; db < NDH; ++db) acc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.f;   // role 0

  // Role 0 waves fetch the K tile, role 1 waves the V tile; tile i goes to stage i % 3.
  KVTiles<HD, HDP, BN> kv;
  kv.init(a, it, t0, nt, role, pair, lane);
  const int n_tiles = kv.n;
  auto issue = [&](int i) { kv.fetch(smem + (i % NST) * 2 * TILE + role * TILE, i); };
  SwWide<HDP> sw;
  sw.init(lane);
  // Every load above has landed before the first DMA (see the head-dim-split kernel).
  dma_wait();
  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);
  // Tile 0 has landed (tile 1's loads, issued after it, may still be in flight).
  if (n_tiles > 1)
    dma_wait_keep<DmaRows<HDP, BN, HD>::kPerWave>();
  else
    dma_wait();
  __syncthreads();

  for (int i = 0; i < n_tiles; ++i) {
    const char *ks = smem + (i % NST) * 2 * TILE;
    const char *vs = ks + TILE;
    char *xp = xbase + ((i & 1) * 4 + pair) * XS;
    h16x8 p0, p1;   // P of the tile (keys 0..15, 16..31 in the operand's order)
    float alpha = 1.f;
    if (role == 0) {
      int nrows, kpos0;
      kv.at(i, nrows, kpos0);
      sw.opaque();
      f32x16 st = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        st = mma16<E>(sw.frag(lds_u32(ks), kc), qf[kc], st);
      reads_ahead<NKC, 1, PA>();   // one fragment read per product, PA products ahead
      const bool need_mask = (nrows < BN) || (kpos0 + BN - 1 > qmin) ||
                             (wl >= 0 && kpos0 < qmax - wl);
      if (need_mask) {
        // Visible keys of this lane's row as a range of tile offsets [lo, hi): inside
        // the tile, causal, and inside the window; compared per element without branches.
        const int lo = (wl >= 0 ? qpos - wl - kpos0 : -BN) - 4 * half;
        const int hi = min(nrows, qpos - kpos0 + 1) - 4 * half;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 8 * (v >> 2) + (v & 3);   // c_row(v, half) - 4 half
          st[v] = ((r >= lo) & (r < hi)) ? st[v] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[v]);
      mx = pair_max(mx) * sf;
      const bool grow = mx > m_run + kSlack;
      if (__any(grow)) {
        alpha = grow ? fast_exp2(m_run - mx) : 1.f;
        if (grow) m_run = mx;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDH; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      uint32_t pw[8];   // P as 16-bit pairs
      float rs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float e0 = fast_exp2(fmaf(st[v], sf, -m_use));
        const float e1 = fast_exp2(fmaf(st[v + 1], sf, -m_use));
        rs += e0;
        rs += e1;
        pw[v / 2] = pack2<E>(e0, e1);
      }
      l_run += rs;
      p0 = words8(pw);
      p1 = words8(pw + 4);
      *reinterpret_cast<uint4 *>(xp + lane * 32) = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      *reinterpret_cast<uint4 *>(xp + lane * 32 + 16) = make_uint4(pw[4], pw[5], pw[6], pw[7]);
      *reinterpret_cast<float *>(xp + 64 * 32 + lane * 4) = alpha;
    }
    // This wave's loads of tile i + 1 have landed (nothing newer is in flight); after the
    // barrier the next stage and every pair's P are visible, and every wave is done with
    // tile i - 1's stage.
    dma_wait();
    __syncthreads();
    if (i + 2 < n_tiles) issue(i + 2);
    if (role == 1) {
      const uint4 w0 = *reinterpret_cast<const uint4 *>(xp + lane * 32);
      const uint4 w1 = *reinterpret_cast<const uint4 *>(xp + lane * 32 + 16);
      p0 = __builtin_bit_cast(h16x8, w0);
      p1 = __builtin_bit_cast(h16x8, w1);
      alpha = *reinterpret_cast<const float *>(xp + 64 * 32 + lane * 4);
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDH; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
      }
    }
    // Oᵀ += Vᵀ Pᵀ over this wave's half of the head dim (blocks past a 192-wide head dim
    // are skipped).
#pragma unroll
    for (int db = 0; db < NDH; ++db) {
      if (HD != HDP && d0 + db * 32 >= HD) continue;
      acc[db] = mma16<E>(sw.trfrag(lds_u32(vs), 0, d0 / 32 + db), p0, acc[db]);
      acc[db] = mma16<E>(sw.trfrag(lds_u32(vs), 16, d0 / 32 + db), p1, acc[db]);
    }
    reads_ahead<2 * NDH, 2, PA>();   // a transposed fragment (two reads) per product, PA ahead
  }

  // Row sums: role 0 holds them (its two lanes of a row a half each) and passes them on,
  // through the P buffer of the parity the last tile did not use (its readers were done
  // before the last barrier).
  float *lx = reinterpret_cast<float *>(xbase + ((n_tiles & 1) * 4 + pair) * XS);
  if (role == 0) {
    const float l = pair_sum(l_run);
    if (half == 0) lx[col] = l;
    if (half == 0 && row_valid)
      a.lse[(long)h * a.lse_ld + seq0 + t0 + tok] = (m_run + fast_log2(l)) * kLn2;
  }
  __syncthreads();
  const float inv = 1.f / lx[col];
  if (row_valid) {
    h16 *optr = reinterpret_cast<h16 *>(a.o) + (long)(seq0 + t0 + tok) * qld + (long)h * HD + d0;
#pragma unroll
    for (int db = 0; db < NDH; ++db) {
      if (HD != HDP && d0 + db * 32 >= HD) continue;   // past a 192-wide head dim
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int dim = db * 32 + 8 * i + 4 * half;
        h16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = rnd<E>(acc[db][4 * i + e] * inv);
        *reinterpret_cast<h16x4 *>(optr + dim) = w;
      }
    }
  }
}

template <typename E, int HD, int HDP>
static hipError_t fwd_wide(const FwdArgs &a, int n, hipStream_t s) {
  if constexpr (HDP == 256)
    hipLaunchKernelGGL((fwd_pair_kernel<E, HD>), dim3(n), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_wide_kernel<E, HD, HDP>), dim3(n), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_wide(int dtype, int hd, const FwdArgs &a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool f = dtype == 2;
  switch (hd) {
    case 256: return f ? fwd_wide<f16, 256, 256>(a, n, s) : fwd_wide<h16, 256, 256>(a, n, s);
    case 512: return f ? fwd_wide<f16, 512, 512>(a, n, s) : fwd_wide<h16, 512, 512>(a, n, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------------ dQ --

template <typename E, int HD, int HDP>
__global__ __launch_bounds__(512, 1) void bwd_dq_wide_kernel(BwdQArgs a) {
  constexpr int BN = 32;
  constexpr int TILE = BN * HDP * 2;     // 32 KB at HDP = 512
  constexpr int NKH = HDP / 2 / 16;
  constexpr int NDQ = HDP / 4 / 32;      // 32-wide output blocks per quarter
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE + 8 * 4096];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // Two groups of four waves, 32 rows each; in a group, role 0 forms partial Sᵀ from
  // Q and role 1 partial dPᵀ from dO, over head-dim half dh.
  const int grp = wave >> 2, wq = wave & 3;
  const int role = wq >> 1, dh = wq & 1;
  float *xch = reinterpret_cast<float *>(smem + 4 * TILE) + grp * 4 * 1024;
  const QItem it = a.items[blockIdx.x];
  const int g = it.g, seq0 = it.seq_start, seqlen = it.seq_len;
  const int t0 = it.tile * a.bm_tok;
  const int nt = min(a.bm_tok, seqlen - t0);
  const int qr = grp * 32 + col;
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

  const int xd0 = dh * (HDP / 2);   // first dim of this wave's half
  const h16 *xptr = reinterpret_cast<const h16 *>(role == 0 ? a.q : a.dout) + qrow * qld +
                     (long)h * HD + xd0;
  // dims past the head dim (padded rows) are zero
  auto real = [&](int kc) { return HD == HDP || xd0 + kc * 16 < HD; };
  h16x8 xf[NKH];
#pragma unroll
  for (int kc = 0; kc < NKH; ++kc)
    xf[kc] = real(kc) ? as_h16x8(*reinterpret_cast<const uint4 *>(xptr + kc * 16 + half * 8))
                      : as_h16x8(make_uint4(0, 0, 0, 0));
  const float sf = a.scale * kLog2e;
  const float lse = a.lse[(long)h * a.lse_ld + qrow];
  const float lse2 = lse * kLog2e;
  // D = rowsum(dO ∘ O) of this lane's row (the preprocess step of the backward, done
  // here): waves 2 / 3 of the group hold dO over the two halves of the head dim; each
  // sums its half against O (the two lanes of a row a quarter each), puts it in the
  // exchange area, and every wave adds the halves 0 + 1 after a barrier.
  if (role == 1) {
    const h16 *optr = reinterpret_cast<const h16 *>(a.o) + qrow * qld + (long)h * HD + xd0;
    float dh_sum = 0.f;
#pragma unroll
    for (int kc = 0; kc < NKH; ++kc) {
      if (!real(kc)) continue;
      const h16x8 o8 = as_h16x8(*reinterpret_cast<const uint4 *>(optr + kc * 16 + half * 8));
#pragma unroll
      for (int e = 0; e < 8; ++e) dh_sum += val<E>(o8[e]) * val<E>(xf[kc][e]);
    }
    dh_sum = pair_sum(dh_sum);
    if (half == 0) xch[dh * 32 + col] = dh_sum;
  }
  __syncthreads();
  const float Dq = xch[col] + xch[32 + col];
  // The dK/dV kernel, which runs next, reads -D and -LSE / scale of every row.
  if (wq == 0 && half == 0 && row_valid) {
    a.Dneg_out[(long)h * a.lse_ld + qrow] = -Dq;
    a.lsn_out[(long)h * a.lse_ld + qrow] = -lse * (1.0f / a.scale);
  }
  const int dq0 = wq * (HDP / 4);

  f32x16 acc[NDQ];
#pragma unroll
  for (int db = 0; db < NDQ; ++db) acc[db] = zero16();

  // Waves 0-3 fetch the K tile, waves 4-7 the V tile; tile i goes to stage i % 2.
  KVTiles<HD, HDP, BN> kv;
  kv.init(a, it, t0, nt, grp, wq, lane);
  const int n_tiles = kv.n;
  auto issue = [&](int i) { kv.fetch(smem + (i & 1) * 2 * TILE + grp * TILE, i); };
  SwWide<HDP> sw;
  sw.init(lane);
  // Every load above has landed before the first DMA: the loop's waits count DMAs only,
  // and no fragment load is left for the compiler to wait on inside the loop (where
  // its wait would drain the next tile's DMA as well).
  dma_wait();
  if (n_tiles > 0) issue(0);

  for (int i = 0; i < n_tiles; ++i) {
    int nrows, kpos0;
    kv.at(i, nrows, kpos0);
    dma_wait();
    __syncthreads();
    if (i + 1 < n_tiles) issue(i + 1);
    const char *ks = smem + (i & 1) * 2 * TILE;
    const char *vs = ks + TILE;

    sw.opaque();
    const char *op = role == 0 ? ks : vs;
    f32x16 part = zero16();
#pragma unroll
    for (int kc = 0; kc < NKH; ++kc)
      part = mma16<E>(sw.frag(lds_u32(op) + dh * HDP, kc), xf[kc], part);
    reads_ahead<NKH, 1, 2>();   // one fragment read per product, two products ahead
    xch_put(xch + wq * 1024, part, lane);
    __syncthreads();
    const bool need_mask = (nrows < BN) || (kpos0 + BN - 1 > qmin) ||
                           (wl >= 0 && kpos0 < qmax - wl);
    // S = partial 0 + partial 1 and dP = partial 2 + partial 3 are formed by the four
    // waves of the group a quad each (C-tile elements 4 wq .. 4 wq + 3): this wave reads
    // quad wq of the four partials, turns it into dS, and writes it as h16 into quad wq
    // of its own slot (which no other wave reads); after a barrier every wave reads the
    // four quads of dS back as its MFMA operand.  The visibility test (keys of this
    // lane's row as tile offsets [lo, hi), compared without branches) is compiled only
    // into the variant for tiles that need it.
    auto grads = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      const int lo = (wl >= 0 ? qpos - wl - kpos0 : -BN) - 4 * half;
      const int hi = min(nrows, qpos - kpos0 + 1) - 4 * half;
      const int q = wq;
      const float4 a0 = xch_quad(xch, q, lane), a1 = xch_quad(xch + 1024, q, lane);
      const float4 b0 = xch_quad(xch + 2048, q, lane), b1 = xch_quad(xch + 3072, q, lane);
      const float st[4] = {a0.x + a1.x, a0.y + a1.y, a0.z + a1.z, a0.w + a1.w};
      const float dpt[4] = {b0.x + b1.x, b0.y + b1.y, b0.z + b1.z, b0.w + b1.w};
      float dsq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = fast_exp2(fmaf(st[e], sf, -lse2));
        if (MASKED) {
          const int r = 8 * q + e;   // c_row(4 q + e, half) - 4 half
          p = ((r >= lo) & (r < hi)) ? p : 0.f;
        }
        dsq[e] = p * (dpt[e] - Dq);
      }
      // 8 bytes per lane, packed (consecutive lanes on consecutive banks)
      *reinterpret_cast<uint2 *>(xch + wq * 1024 + q * 256 + lane * 2) =
          make_uint2(pack2<E>(dsq[0], dsq[1]), pack2<E>(dsq[2], dsq[3]));
    };
    if (need_mask)
      grads(std::true_type{});
    else
      grads(std::false_type{});
    __syncthreads();
    uint2 dd[4];   // quad w of slot w: dS of elements 4w .. 4w+3
#pragma unroll
    for (int w = 0; w < 4; ++w)
      dd[w] = *reinterpret_cast<const uint2 *>(xch + w * 1024 + w * 256 + lane * 2);
    const h16x8 d0 = __builtin_bit_cast(h16x8, make_uint4(dd[0].x, dd[0].y, dd[1].x, dd[1].y));
    const h16x8 d1 = __builtin_bit_cast(h16x8, make_uint4(dd[2].x, dd[2].y, dd[3].x, dd[3].y));
    // dQᵀ += Kᵀ dSᵀ over this wave's quarter of the head dim (column blocks counted
    // from the tile's start: a quarter of a 256-wide row starts inside a swizzle group).
#pragma unroll
    for (int db = 0; db < NDQ; ++db) {
      acc[db] = mma16<E>(sw.trfrag(lds_u32(ks), 0, dq0 / 32 + db), d0, acc[db]);
      acc[db] = mma16<E>(sw.trfrag(lds_u32(ks), 16, dq0 / 32 + db), d1, acc[db]);
    }
    reads_ahead<2 * NDQ, 2, 2>();   // a transposed fragment (two reads) per product, two ahead
  }

  if (row_valid) {
    h16 *optr = reinterpret_cast<h16 *>(a.dq) + qrow * qld + (long)h * HD + dq0;
#pragma unroll
    for (int db = 0; db < NDQ; ++db) {
      if (HD != HDP && dq0 + db * 32 >= HD) continue;   // padded dims: not stored
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
}

// dQ at HDP = 256 (head dims 192 and 256): 128 query rows per workgroup of 8 waves,
// four pairs of 32 rows.  In pair p, wave p (role 0) holds Q of the pair's rows over the
// whole head dim and forms Sᵀ = K Qᵀ; wave p + 4 (role 1, on the same SIMD) holds dO and
// forms dPᵀ = V dOᵀ.  Each writes its tile to LDS, and after one barrier both read the
// two tiles back, form dSᵀ for the whole tile and accumulate dQ over their half of the
// head dim.  Three K / V stages and a double-buffered tile area let that one barrier
// per key tile also hand over the next stage (each wave waits for its own loads of
// tile i + 1 first; the stage of tile i - 1, finished by every wave at the barrier of
// tile i, takes tile i + 2).
template <typename E, int HD>
__global__ __launch_bounds__(512, 1) void bwd_dq_pair_kernel(BwdQArgs a) {
  constexpr int HDP = 256;
  constexpr int BN = 32;
  constexpr int TILE = BN * HDP * 2;     // 16 KB
  constexpr int NKC = HD / 16;           // k-steps over the real head dim
  constexpr int NDH = HDP / 2 / 32;      // 32-wide output blocks per half of the head dim
  constexpr int NST = 3;
  constexpr int PA = 2;                  // fragment reads ahead of the products
  static_assert(HD == 192 || HD == 256, "head dims staged in 256-wide rows");
  __shared__ __attribute__((aligned(16))) char smem[NST * 2 * TILE + 2 * 8 * 4096];
  float *tbuf = reinterpret_cast<float *>(smem + NST * 2 * TILE);   // [2][wave] 32 x 32 tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int role = wave >> 2, pair = wave & 3;
  const QItem it = a.items[blockIdx.x];
  const int g = it.g, seq0 = it.seq_start, seqlen = it.seq_len;
  const int t0 = it.tile * a.bm_tok;
  const int nt = min(a.bm_tok, seqlen - t0);
  const int qr = pair * 32 + col;
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

  const h16 *xptr = reinterpret_cast<const h16 *>(role == 0 ? a.q : a.dout) + qrow * qld + (long)h * HD;
  h16x8 xf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    xf[kc] = as_h16x8(*reinterpret_cast<const uint4 *>(xptr + kc * 16 + half * 8));
  const float sf = a.scale * kLog2e;
  const float lse = a.lse[(long)h * a.lse_ld + qrow];
  const float lse2 = lse * kLog2e;
  // D = rowsum(dO ∘ O) of this lane's row (the backward's preprocess, done here): the
  // dO-holding wave sums the row against O (the two lanes of a row half each) and
  // passes it to its partner through LDS.
  float *dx = tbuf + pair * 32;
  if (role == 1) {
    const h16 *optr = reinterpret_cast<const h16 *>(a.o) + qrow * qld + (long)h * HD;
    float dsum = 0.f;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const h16x8 o8 = as_h16x8(*reinterpret_cast<const uint4 *>(optr + kc * 16 + half * 8));
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += val<E>(o8[e]) * val<E>(xf[kc][e]);
    }
    dsum = pair_sum(dsum);
    if (half == 0) dx[col] = dsum;
  }
  __syncthreads();
  const float Dq = dx[col];
  // The dK/dV kernel, which runs next, reads -D and -LSE / scale of every row.
  if (role == 1 && half == 0 && row_valid) {
    a.Dneg_out[(long)h * a.lse_ld + qrow] = -Dq;
    a.lsn_out[(long)h * a.lse_ld + qrow] = -lse * (1.0f / a.scale);
  }
  const int dq0 = role * (HDP / 2);   // first dim of this wave's half of dQ

  f32x16 acc[NDH];
#pragma unroll
  for (int db = 0; db < NDH; ++db) acc[db] = zero16();

  // Role 0 waves fetch the K tile, role 1 waves the V tile; tile i goes to stage i % 3.
  KVTiles<HD, HDP, BN> kv;
  kv.init(a, it, t0, nt, role, pair, lane);
  const int n_tiles = kv.n;
  auto issue = [&](int i) { kv.fetch(smem + (i % NST) * 2 * TILE + role * TILE, i); };
  SwWide<HDP> sw;
  sw.init(lane);
  // Every load above has landed before the first DMA (see the head-dim-split kernel).
  dma_wait();
  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);
  // Tile 0 has landed (tile 1's loads, issued after it, may still be in flight).
  if (n_tiles > 1)
    dma_wait_keep<DmaRows<HDP, BN, HD>::kPerWave>();
  else
    dma_wait();
  __syncthreads();

  for (int i = 0; i < n_tiles; ++i) {
    int nrows, kpos0;
    kv.at(i, nrows, kpos0);
    const char *ks = smem + (i % NST) * 2 * TILE;
    float *tb = tbuf + (i & 1) * 8 * 1024;
    {   // Sᵀ (role 0) or dPᵀ (role 1) over the whole head dim, into this wave's slot
      sw.opaque();
      const char *op = ks + role * TILE;
      f32x16 part = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        part = mma16<E>(sw.frag(lds_u32(op), kc), xf[kc], part);
      reads_ahead<NKC, 1, PA>();   // one fragment read per product, PA products ahead
      xch_put(tb + wave * 1024, part, lane);
    }
    // This wave's loads of tile i + 1 have landed (nothing newer is in flight); after the
    // barrier the next stage and both tiles of every pair are visible, and every wave is
    // done with tile i - 1's stage.
    dma_wait();
    __syncthreads();
    if (i + 2 < n_tiles) issue(i + 2);
    const bool need_mask = (nrows < BN) || (kpos0 + BN - 1 > qmin) ||
                           (wl >= 0 && kpos0 < qmax - wl);
    // dSᵀ = P (dPᵀ - D) of the whole tile (both waves of the pair form the same values);
    // the visibility test (keys of this lane's row as tile offsets [lo, hi)) is
    // compiled only into the variant for tiles that need it.
    const float *st = tb + pair * 1024, *dp = tb + (pair + 4) * 1024;
    h16x8 d0, d1;
    auto grads = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      const int lo = (wl >= 0 ? qpos - wl - kpos0 : -BN) - 4 * half;
      const int hi = min(nrows, qpos - kpos0 + 1) - 4 * half;
      float dsv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 s4 = xch_quad(st, q, lane), p4 = xch_quad(dp, q, lane);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w}, pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p = fast_exp2(fmaf(sv[e], sf, -lse2));
          if (MASKED) {
            const int r = 8 * q + e;   // c_row(4 q + e, half) - 4 half
            p = ((r >= lo) & (r < hi)) ? p : 0.f;
          }
          dsv[4 * q + e] = p * (pv[e] - Dq);
        }
      }
      d0 = pack8<E>(dsv);
      d1 = pack8<E>(dsv + 8);
    };
    if (need_mask)
      grads(std::true_type{});
    else
      grads(std::false_type{});
    // dQᵀ += Kᵀ dSᵀ over this wave's half of the head dim (column blocks counted from
    // the tile's start; blocks past a 192-wide head dim are skipped).
#pragma unroll
    for (int db = 0; db < NDH; ++db) {
      if (HD != HDP && dq0 + db * 32 >= HD) continue;
      acc[db] = mma16<E>(sw.trfrag(lds_u32(ks), 0, dq0 / 32 + db), d0, acc[db]);
      acc[db] = mma16<E>(sw.trfrag(lds_u32(ks), 16, dq0 / 32 + db), d1, acc[db]);
    }
    reads_ahead<2 * NDH, 2, PA>();   // a transposed fragment (two reads) per product, PA ahead
  }

  if (row_valid) {
    h16 *optr = reinterpret_cast<h16 *>(a.dq) + qrow * qld + (long)h * HD + dq0;
#pragma unroll
    for (int db = 0; db < NDH; ++db) {
      if (HD != HDP && dq0 + db * 32 >= HD) continue;   // past a 192-wide head dim
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
}

template <typename E, int HD, int HDP>
static hipError_t dq_wide(const BwdQArgs &a, int n, hipStream_t s) {
  if constexpr (HDP == 256)
    hipLaunchKernelGGL((bwd_dq_pair_kernel<E, HD>), dim3(n), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_wide_kernel<E, HD, HDP>), dim3(n), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_wide(int dtype, int hd, const BwdQArgs &a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool f = dtype == 2;
  switch (hd) {
    case 192: return f ? dq_wide<f16, 192, 256>(a, n, s) : dq_wide<h16, 192, 256>(a, n, s);
    case 256: return f ? dq_wide<f16, 256, 256>(a, n, s) : dq_wide<h16, 256, 256>(a, n, s);
    case 512: return f ? dq_wide<f16, 512, 512>(a, n, s) : dq_wide<h16, 512, 512>(a, n, s);
    default: return hipErrorInvalidValue;
  }
}

// --------------------------------------------------------------------- dK/dV --

// MAP: the q-heads of the kv head come from the GQA head table (a.qhead).
template <typename E, int HD, int HDP, bool MAP>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_wide_kernel(BwdKVArgs a) {
  constexpr int BM = 32;                 // query rows per step
  constexpr int TILE = BM * HDP * 2;     // 32 KB at HDP = 512
  constexpr int NKH = HDP / 2 / 16;
  constexpr int NDQ = HDP / 4 / 32;
  constexpr int RPB = 1024 / (HDP * 2);  // staged rows per 1 KB DMA block (1 or 2)
  constexpr int CPR = HDP / 8;           // 16-byte chunks per staged row
  constexpr int NIW = BM / RPB / 4;      // DMA instructions of each wave per step
  constexpr int STAGE = 2 * TILE;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE + 8 * 4096];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // Two groups of four waves, 32 keys each; in a group, role 0 forms partial S with K
  // and role 1 partial dP with V, over head-dim half dh.
  const int grp = wave >> 2, wq = wave & 3;
  const int role = wq >> 1, dh = wq & 1;
  float *xch = reinterpret_cast<float *>(smem + 2 * STAGE) + grp * 4 * 1024;
  const KVItem it = a.items[blockIdx.x];
  const int g = it.g, G = a.G, P = it.ctx_len, wl = a.window_left;
  const bool ctx = it.region == kRegionCtx;
  const long qld = (long)a.Hq * HD;
  const long kld = (long)a.Hkv * HD;
  const int own0 = ctx ? it.ctx_start : sload_i32(a.cu, it.seq_lo);
  const int nkeys = ctx ? P - it.key_start : sload_i32(a.cu, it.seq_lo + 1) - own0 - it.key_start;
  const int kbase = ctx ? 0 : P;
  const int nk_tile = min(kBwdBNWide, nkeys);
  const int gk0 = grp * 32;              // the group's first key in the tile
  const int nkeys_g = nkeys - gk0;       // keys of the tile this group holds (may be <= 0)

  const int key = gk0 + col;
  const bool key_valid = key < nkeys;
  const float sf = a.scale * kLog2e;
  // K (role 0) or V (role 1) rows of the group's keys, this wave's head-dim half;
  // keys past the tile's end read as zeros (buffer range check).
  const int xd0 = dh * (HDP / 2);   // first dim of this wave's half
  const h16 *xp = reinterpret_cast<const h16 *>(
                       role == 0 ? (ctx ? a.k_ctx : a.k_own) : (ctx ? a.v_ctx : a.v_own)) +
                   (long)(own0 + it.key_start + gk0) * kld + (long)g * HD + xd0;
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc_u(xp, nkeys_g > 0 ? (uint32_t)nkeys_g * (uint32_t)(kld * 2) : 0u);
  h16x8 xf[NKH];
#pragma unroll
  for (int kc = 0; kc < NKH; ++kc)   // dims past the head dim (padded rows) are zero
    xf[kc] = (HD == HDP || xd0 + kc * 16 < HD)
                 ? __builtin_bit_cast(h16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rk, col * (int)(kld * 2) + (kc * 16 + half * 8) * 2, 0, 0))
                 : as_h16x8(make_uint4(0, 0, 0, 0));
  const int kpos = kbase + it.key_start + key;
  const int f_vis_lo = key_valid ? max(0, (kpos - P) * G) : 0x7fffffff;
  const int f_vis_hi = (wl >= 0) ? max(0, (kpos + wl - P + 1) * G) : 0x7fffffff;
  const int dq0 = wq * (HDP / 4);

  f32x16 dk[NDQ], dv[NDQ];
#pragma unroll
  for (int db = 0; db < NDQ; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  // Steps of BM flattened rows, walked from the last one backward.
  RowSteps<BM> rs;
  rs.init(a.cu, it, nk_tile, P, wl, G, ctx, kBwdBNWide);

  const int qld_b = (int)(qld * 2);
  const int head0_b = g * G * HD * 2;
  HeadMap hm;
  if constexpr (MAP) hm.init(a.qhead, g, G, lane);
  const int r4 = 4 % G;                                  // head step of 4 flattened rows
  const int step4 = (4 / G) * qld_b + r4 * (HD * 2);     // their byte step before a wrap
  // Waves 0-3 fetch the step's Q rows, waves 4-7 its dO rows: 1 KB block b of the step's
  // tile (staged rows RPB b .. RPB b + RPB - 1, flattened (token, head) rows) is
  // written by wave b % 4.
  // ceil(2^24 / G): r * g_recip >> 24 is r / G exactly for r < 64 and G <= 128.
  const uint32_t g_recip = __builtin_amdgcn_readfirstlane(((1u << 24) + (uint32_t)G - 1) / (uint32_t)G);
  const h16 *xsrc = reinterpret_cast<const h16 *>(grp ? a.dout : a.q);
  // The first head-dim half of each role starts its partial at -LSE / scale (scores)
  // or -D (dP) of the step's rows: lane l fetches row l % 32's value into a register
  // one step ahead, and the wave spreads it over the C layout with ds_bpermute.
  const __amdgpu_buffer_rsrc_t r_ld = make_rsrc_u(role == 0 ? (const void *)a.lsn : (const void *)a.Dneg,
                                                  (uint32_t)((long)a.Hq * a.lse_ld * 4));
  auto issue = [&](char *st) {
    const int s0 = rs.cs0;
    const int len = rs.clen;
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc_u(xsrc + (long)s0 * qld, (uint32_t)len * (uint32_t)qld_b);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_u32(st + grp * TILE) + wq * 1024);
    if constexpr (RPB == 1) {
      // One row per block, wave-uniform: (token, head) of the wave's first row, then
      // stepped 4 rows at a time without a division.
      const int f = rs.cf + wq;
      int t = (int)((unsigned)f / (unsigned)G);
      int j = f - t * G;
      int roff = t * qld_b + head0_b + j * (HD * 2);
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        const int r = k * 4 + wq;
        // With a head table the row's head (wave-uniform) comes from the table.
        const int ro = MAP ? roff - head0_b - j * (HD * 2) + hm.at_uniform(j) * (HD * 2) : roff;
        dma16(rx, l0 + k * 4096, ro + ((lane ^ Swz<HDP>::swz(r)) << 4));
        // 4 rows on: q4 tokens and r4 heads, plus one token when the head index wraps
        j += r4;
        roff += step4;
        if (j >= G) {
          j -= G;
          roff += qld_b - G * HD * 2;
        }
      }
    } else {
      // RPB rows per block: lane l fills chunk slot l % CPR of row RPB b + l / CPR, with
      // the source chunk that the swizzle puts there (zeros past the head dim).
      const int ft = rs.cf / G, fj = rs.cf - ft * G;
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        const int r = RPB * (k * 4 + wq) + lane / CPR;
        const int tr_ = (int)(((uint32_t)r * g_recip) >> 24);   // r / G (r < 64)
        int t = ft + tr_, j = fj + (r - tr_ * G);
        if (j >= G) {
          j -= G;
          ++t;
        }
        const int hoff = MAP ? hm.at(j, G) * (HD * 2) : head0_b + j * (HD * 2);
        const int src = (lane % CPR) ^ Swz<HDP>::swz(r);
        const int off = (HD == HDP || src < HD / 8) ? t * qld_b + hoff + (src << 4) : 0x7ffffff0;
        dma16(rx, l0 + k * 4096, off);
      }
    }
  };
  // Row init values of the step at the cursor (rows past the sequence read 0 and are
  // masked later).
  auto fetch_init = [&]() -> float {
    const int s0 = rs.cs0;
    const int f = rs.cf + col;
    const int t = (int)((unsigned)f / (unsigned)G), j = f - t * G;
    const int hq = MAP ? hm.at(j, G) : g * G + j;
    const int off = (hq * a.lse_ld + s0 + t) * 4;
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_ld, off, 0, 0));
  };

  SwWide<HDP> sw;
  sw.init(lane);
  // Every load above has landed before the first DMA (see the dQ kernel).
  dma_wait();
  int stage = 0;
  bool have = !rs.done;
  int f0 = 0, flo = 0, fend = 0;   // the step at hand
  float xinit = 0.f;
  if (have) {
    issue(smem);
    if (dh == 0) xinit = fetch_init();
    rs.advance(f0, flo, fend);
  }

  const int kpa = kbase + it.key_start + gk0;
  const int kpb = kpa + 31;
  while (have) {
    f32x16 part = zero16();
    // The partial's start values (waits for this step's fetches, which the barrier
    // below needs anyway).
    if (dh == 0) {
      const int xi = __builtin_bit_cast(int, xinit);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        part[v] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(c_row(v, half) << 2, xi));
    }
    dma_wait();
    __syncthreads();
    const bool more = !rs.done;
    int g0 = 0, glo = 0, gend = 0;
    if (more) {   // every wave is done with the stage of the previous step
      issue(smem + (stage ^ 1) * STAGE);
      if (dh == 0) xinit = fetch_init();
      rs.advance(g0, glo, gend);
    }
    const char *qs = smem + stage * STAGE;
    const char *dos = qs + TILE;
    sw.opaque();

    const char *op = role == 0 ? qs : dos;
#pragma unroll
    for (int kc = 0; kc < NKH; ++kc)
      part = mma16<E>(sw.frag(lds_u32(op) + dh * HDP, kc), xf[kc], part);
    reads_ahead<NKH, 1, 2>();   // one fragment read per product, two products ahead
    xch_put(xch + wq * 1024, part, lane);
    __syncthreads();

    // Every row of the block sees every key of the group: the last key is causal for
    // the first row's token (kpb - P <= flo / G) and the first key is inside the last
    // row's window (kpa >= P + (fend - 1) / G - wl), in flattened units.
    const bool full = (f0 >= flo) && (f0 + BM <= fend) && (32 <= nkeys_g) &&
                      ((kpb - P) * G <= flo) && (wl < 0 || fend <= (kpa - P + wl + 1) * G);
    // S = partial 0 + partial 1 and dP - D = partial 2 + partial 3 are formed by the four
    // waves of the group a quad each (C-tile elements 4 wq .. 4 wq + 3): this wave reads
    // quad wq of the four partials, turns it into P and dS, and writes them as h16 into
    // quad wq of its own slot (which no other wave reads); after a barrier every wave
    // reads the four quads of P and dS back as its MFMA operands.  The visibility test
    // is compiled only into the variant for blocks that straddle a mask edge or a range
    // end.
    auto probs = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      const int lo = max(flo, f_vis_lo) - f0 - 4 * half;   // visible row offsets [lo, hi)
      const int hi = min(fend, f_vis_hi) - f0 - 4 * half;
      const int q = wq;
      const float4 a0 = xch_quad(xch, q, lane), a1 = xch_quad(xch + 1024, q, lane);
      const float4 b0 = xch_quad(xch + 2048, q, lane), b1 = xch_quad(xch + 3072, q, lane);
      const float st[4] = {a0.x + a1.x, a0.y + a1.y, a0.z + a1.z, a0.w + a1.w};
      const float dpt[4] = {b0.x + b1.x, b0.y + b1.y, b0.z + b1.z, b0.w + b1.w};
      float pq[4], dq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = fast_exp2(st[e] * sf);
        if (MASKED) {
          const int r = 8 * q + e;
          p = ((r >= lo) & (r < hi)) ? p : 0.f;
        }
        pq[e] = p;
        dq[e] = p * dpt[e];
      }
      *reinterpret_cast<uint4 *>(xch + wq * 1024 + q * 256 + lane * 4) =
          make_uint4(pack2<E>(pq[0], pq[1]), pack2<E>(pq[2], pq[3]), pack2<E>(dq[0], dq[1]),
                     pack2<E>(dq[2], dq[3]));
    };
    if (full)
      probs(std::false_type{});
    else
      probs(std::true_type{});
    __syncthreads();
    uint4 pd[4];   // quad w of slot w: P of elements 4w .. 4w+3 (x, y), dS (z, w)
#pragma unroll
    for (int w = 0; w < 4; ++w)
      pd[w] = *reinterpret_cast<const uint4 *>(xch + w * 1024 + w * 256 + lane * 4);
    const h16x8 p0 = __builtin_bit_cast(h16x8, make_uint4(pd[0].x, pd[0].y, pd[1].x, pd[1].y));
    const h16x8 p1 = __builtin_bit_cast(h16x8, make_uint4(pd[2].x, pd[2].y, pd[3].x, pd[3].y));
    const h16x8 s0 = __builtin_bit_cast(h16x8, make_uint4(pd[0].z, pd[0].w, pd[1].z, pd[1].w));
    const h16x8 s1 = __builtin_bit_cast(h16x8, make_uint4(pd[2].z, pd[2].w, pd[3].z, pd[3].w));
    // dV += Pᵀ dO and dK += dSᵀ Q over this wave's quarter of the head dim.
#pragma unroll
    for (int db = 0; db < NDQ; ++db) {
      const int cb = dq0 / 32 + db;   // column block counted from the tile's start
      dv[db] = mma16<E>(p0, sw.trfrag(lds_u32(dos), 0, cb), dv[db]);
      dv[db] = mma16<E>(p1, sw.trfrag(lds_u32(dos), 16, cb), dv[db]);
      dk[db] = mma16<E>(s0, sw.trfrag(lds_u32(qs), 0, cb), dk[db]);
      dk[db] = mma16<E>(s1, sw.trfrag(lds_u32(qs), 16, cb), dk[db]);
    }
    reads_ahead<4 * NDQ, 2, 2>();   // a transposed fragment (two reads) per product, two ahead
    have = more;
    f0 = g0, flo = glo, fend = gend;
    stage ^= 1;
  }

  const bool to_acc = ctx || a.own_to_acc;
#pragma unroll
  for (int db = 0; db < NDQ; ++db) {
    if (HD != HDP && dq0 + db * 32 >= HD) continue;   // padded dims: not stored
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = gk0 + c_row(v, half);
      if (k >= nkeys) continue;
      const long off = (long)(own0 + it.key_start + k) * kld + (long)g * HD + dq0 + db * 32 + col;
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
}

// dK/dV at HDP = 256 (head dims 192 and 256): 128 keys per workgroup of 8 waves, four
// pairs of 32 keys.  In pair p, wave p (role 0) holds K of the pair's keys over the
// whole head dim and forms S, P and dV; wave p + 4 (role 1, on the same SIMD) holds V
// and forms dP, dS and dK.  P crosses from role 0 to role 1 through LDS in fp32, so
// dS = P (dP - D) is formed as in the other kernels.  Each wave accumulates one
// gradient over the whole head dim (128 registers).  Three Q / dO stages (each with the
// rows' -LSE / scale and -D as DMA words) and a double-buffered P area let one barrier
// per step both hand over the next stage and pass P: every wave waits for its own loads
// of step i + 1 before the barrier of step i, and the stage of step i - 1, which all
// waves have finished with by then, takes step i + 2.
template <typename E, int HD, bool MAP>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_kernel(BwdKVArgs a) {
  constexpr int HDP = 256;
  constexpr int BM = 32;                 // query rows per step
  constexpr int TILE = BM * HDP * 2;     // 16 KB
  constexpr int NKC = HD / 16;           // k-steps over the real head dim
  constexpr int NDB = HD / 32;           // real 32-wide output blocks
  constexpr int RPB = 2;                 // staged rows per 1 KB DMA block
  constexpr int CPR = HDP / 8;           // 16-byte chunks per staged row
  constexpr int NIW = BM / RPB / 4;      // DMA instructions of each wave per step
  constexpr int NST = 3;
  constexpr int STAGE = 2 * TILE + 512;  // Q, dO, then 64 words each of -LSE / scale and -D
  static_assert(HD == 192 || HD == 256, "head dims staged in 256-wide rows");
  constexpr int PA = 2;   // fragment reads ahead of the products
  __shared__ __attribute__((aligned(16))) char smem[NST * STAGE + 2 * 4 * 4096];
  float *pbuf = reinterpret_cast<float *>(smem + NST * STAGE);   // [2][pair] 32 x 32 P tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int role = wave >> 2, pair = wave & 3;
  const KVItem it = a.items[blockIdx.x];
  const int g = it.g, G = a.G, P = it.ctx_len, wl = a.window_left;
  const bool ctx = it.region == kRegionCtx;
  const long qld = (long)a.Hq * HD;
  const long kld = (long)a.Hkv * HD;
  const int own0 = ctx ? it.ctx_start : sload_i32(a.cu, it.seq_lo);
  const int nkeys = ctx ? P - it.key_start : sload_i32(a.cu, it.seq_lo + 1) - own0 - it.key_start;
  const int kbase = ctx ? 0 : P;
  const int nk_tile = min(kBwdBNPair, nkeys);
  const int gk0 = pair * 32;             // the pair's first key in the tile
  const int nkeys_g = nkeys - gk0;       // keys of the tile this pair holds (may be <= 0)

  const int key = gk0 + col;
  const bool key_valid = key < nkeys;
  const float sf = a.scale * kLog2e;
  // K (role 0) or V (role 1) rows of the pair's keys over the whole head dim; keys past
  // the tile's end read as zeros (buffer range check).
  const h16 *xp = reinterpret_cast<const h16 *>(
                       role == 0 ? (ctx ? a.k_ctx : a.k_own) : (ctx ? a.v_ctx : a.v_own)) +
                   (long)(own0 + it.key_start + gk0) * kld + (long)g * HD;
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc_u(xp, nkeys_g > 0 ? (uint32_t)nkeys_g * (uint32_t)(kld * 2) : 0u);
  h16x8 xf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    xf[kc] = __builtin_bit_cast(h16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                           rk, col * (int)(kld * 2) + (kc * 16 + half * 8) * 2, 0, 0));
  const int kpos = kbase + it.key_start + key;
  const int f_vis_lo = key_valid ? max(0, (kpos - P) * G) : 0x7fffffff;
  const int f_vis_hi = (wl >= 0) ? max(0, (kpos + wl - P + 1) * G) : 0x7fffffff;

  f32x16 acc[NDB];   // dV (role 0) or dK (role 1) of the pair's keys
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  // Steps of BM flattened rows, walked from the last one backward.
  RowSteps<BM> rs;
  rs.init(a.cu, it, nk_tile, P, wl, G, ctx, 0);

  const int qld_b = (int)(qld * 2);
  const int head0_b = g * G * HD * 2;
  HeadMap hm;
  if constexpr (MAP) hm.init(a.qhead, g, G, lane);
  // ceil(2^24 / G): r * g_recip >> 24 is r / G exactly for r < 64 and G <= 128.
  const uint32_t g_recip = __builtin_amdgcn_readfirstlane(((1u << 24) + (uint32_t)G - 1) / (uint32_t)G);
  const h16 *xsrc = reinterpret_cast<const h16 *>(role ? a.dout : a.q);
  // Role 0 waves fetch the step's Q rows, role 1 waves its dO rows: 1 KB block b of a
  // tile (staged rows 2 b and 2 b + 1) is written by the wave of pair b % 4.  The first
  // wave of each role also fetches its rows' -LSE / scale (role 0) or -D (role 1).
  const __amdgpu_buffer_rsrc_t r_init = make_rsrc_u(role == 0 ? (const void *)a.lsn : (const void *)a.Dneg,
                                                    (uint32_t)((long)a.Hq * a.lse_ld * 4));
  auto issue = [&](char *st) {
    const int s0 = rs.cs0;
    const int len = rs.clen;
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc_u(xsrc + (long)s0 * qld, (uint32_t)len * (uint32_t)qld_b);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_u32(st + role * TILE) + pair * 1024);
    const int ft = rs.cf / G, fj = rs.cf - ft * G;
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
      const int r = RPB * (k * 4 + pair) + lane / CPR;
      const int tr_ = (int)(((uint32_t)r * g_recip) >> 24);   // r / G (r < 64)
      int t = ft + tr_, j = fj + (r - tr_ * G);
      if (j >= G) {
        j -= G;
        ++t;
      }
      const int hoff = MAP ? hm.at(j, G) * (HD * 2) : head0_b + j * (HD * 2);
      const int src = (lane % CPR) ^ Swz<HDP>::swz(r);
      const int off = (HD == HDP || src < HD / 8) ? t * qld_b + hoff + (src << 4) : 0x7ffffff0;
      dma16(rx, l0 + k * 4096, off);
    }
    if (pair == 0) {   // lane l < 32 fetches row l's word, the other lanes zeros
      const int f = rs.cf + lane;
      const int t = (int)((unsigned)f / (unsigned)G), j = f - t * G;
      const int hq = MAP ? hm.at(j & 63, G) : g * G + j;   // j < G for every lane
      const int off = lane < BM ? (hq * a.lse_ld + s0 + t) * 4 : 0x7fffffff;
      dma4(r_init, __builtin_amdgcn_readfirstlane(lds_u32(st + 2 * TILE) + role * 256), off);
    }
  };

  SwWide<HDP> sw;
  sw.init(lane);
  // Every load above has landed before the first DMA (see the dQ kernel).
  dma_wait();
  int stage = 0, pb = 0;
  bool have = !rs.done;
  int f0 = 0, flo = 0, fend = 0;   // the step at hand
  bool have1 = false;              // the next step, already in flight
  int h0 = 0, hlo = 0, hend = 0;
  if (have) {
    issue(smem);
    rs.advance(f0, flo, fend);
    have1 = !rs.done;
    if (have1) {
      issue(smem + STAGE);
      rs.advance(h0, hlo, hend);
    }
  }
  // Step 0 has landed (step 1's loads, issued after it, may still be in flight).
  if (have1) {
    if (pair == 0)
      dma_wait_keep<NIW + 1>();
    else
      dma_wait_keep<NIW>();
  } else {
    dma_wait();
  }
  __syncthreads();

  const int kpa = kbase + it.key_start + gk0;
  const int kpb = kpa + 31;
  while (have) {
    const char *qs = smem + stage * STAGE;
    const char *dos = qs + TILE;
    float *pt = pbuf + (pb * 4 + pair) * 1024;
    // Scores (role 0) or dP (role 1) of the pair's keys over the whole head dim, started
    // at -LSE / scale or -D of the rows (C layout: rows 8 i + 4 half .. + 3).
    auto product = [&]() {
      f32x16 part;
      const float *ini = reinterpret_cast<const float *>(qs + 2 * TILE) + role * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = *reinterpret_cast<const float4 *>(ini + 8 * i + 4 * half);
        part[4 * i] = x.x, part[4 * i + 1] = x.y, part[4 * i + 2] = x.z, part[4 * i + 3] = x.w;
      }
      sw.opaque();
      const char *op = role == 0 ? qs : dos;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        part = mma16<E>(sw.frag(lds_u32(op), kc), xf[kc], part);
      reads_ahead<NKC, 1, PA>();   // one fragment read per product, PA products ahead
      return part;
    };
    h16x8 x0, x1;   // P (role 0) or dS (role 1), rows 0..15 and 16..31 of the step
    if (role == 0) {
      // S, then P; the visibility test is compiled only into the variant for steps that
      // straddle a mask edge or a range end.  Every row of the step sees every key of
      // the pair when the step lies inside the causal and window bounds of both its
      // first and last key.
      const f32x16 st = product();
      const bool full = (f0 >= flo) && (f0 + BM <= fend) && (32 <= nkeys_g) &&
                        ((kpb - P) * G <= flo) && (wl < 0 || fend <= (kpa - P + wl + 1) * G);
      float pv[16];
      auto probs = [&](auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
        const int lo = max(flo, f_vis_lo) - f0 - 4 * half;   // visible row offsets [lo, hi)
        const int hi = min(fend, f_vis_hi) - f0 - 4 * half;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p = fast_exp2(st[v] * sf);
          if (MASKED) {
            const int r = 8 * (v >> 2) + (v & 3);   // c_row(v, half) - 4 half
            p = ((r >= lo) & (r < hi)) ? p : 0.f;
          }
          pv[v] = p;
        }
      };
      if (full)
        probs(std::false_type{});
      else
        probs(std::true_type{});
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(pt + q * 256 + lane * 4) =
            make_float4(pv[4 * q], pv[4 * q + 1], pv[4 * q + 2], pv[4 * q + 3]);
      x0 = pack8<E>(pv);   // packed before the barrier: only these cross it
      x1 = pack8<E>(pv + 8);
    }
    // This wave's loads of the next step have landed (nothing newer is in flight); after
    // the barrier the next stage and this step's P are visible to every wave, and every
    // wave is done with the previous step's stage.
    dma_wait();
    __syncthreads();
    const bool more = !rs.done;
    int g0 = 0, glo = 0, gend = 0;
    if (more) {
      issue(smem + (stage == 0 ? 2 : stage - 1) * STAGE);
      rs.advance(g0, glo, gend);
    }
    if (role == 1) {
      // dP - D after the barrier (so it is not held across it), then dS = P (dP - D)
      const f32x16 dpt = product();
      float dsv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 p4 = xch_quad(pt, q, lane);
        dsv[4 * q] = p4.x * dpt[4 * q];
        dsv[4 * q + 1] = p4.y * dpt[4 * q + 1];
        dsv[4 * q + 2] = p4.z * dpt[4 * q + 2];
        dsv[4 * q + 3] = p4.w * dpt[4 * q + 3];
      }
      x0 = pack8<E>(dsv);
      x1 = pack8<E>(dsv + 8);
    }
    // dV += Pᵀ dO (role 0) or dK += dSᵀ Q (role 1) over the whole head dim.
    const char *bs = role == 0 ? dos : qs;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      acc[db] = mma16<E>(x0, sw.trfrag(lds_u32(bs), 0, db), acc[db]);
      acc[db] = mma16<E>(x1, sw.trfrag(lds_u32(bs), 16, db), acc[db]);
    }
    reads_ahead<2 * NDB, 2, PA>();   // a transposed fragment (two reads) per product, PA ahead
    have = have1;
    have1 = more;
    f0 = h0, flo = hlo, fend = hend;
    h0 = g0, hlo = glo, hend = gend;
    stage = stage == 2 ? 0 : stage + 1;
    pb ^= 1;
  }

  const bool to_acc = ctx || a.own_to_acc;
  const float gs = role == 0 ? 1.f : a.scale;   // dK carries the softmax scale
  float *acc_out = role == 0 ? a.acc_dv : a.acc_dk;
  float *split_out = role == 0 ? a.split_dv : a.split_dk;
  h16 *own_out = reinterpret_cast<h16 *>(role == 0 ? a.dv_own : a.dk_own);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = gk0 + c_row(v, half);
      if (k >= nkeys) continue;
      const long off = (long)(own0 + it.key_start + k) * kld + (long)g * HD + db * 32 + col;
      const float gv = acc[db][v] * gs;
      if (ctx && a.split_dk) {   // split mode: the chunk's own slice, one writer
        split_out[(long)(it.seq_lo / a.split_chunk) * a.split_stride + off] = gv;
      } else if (to_acc) {
        atomicAdd(acc_out + off, gv);
      } else {
        own_out[off] = rnd<E>(gv);
      }
    }
  }
}

template <typename E, int HD, int HDP>
static hipError_t dkdv_wide(const BwdKVArgs &a, int n, hipStream_t s) {
  if constexpr (HDP == 256) {
    if (a.qhead)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<E, HD, true>), dim3(n), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<E, HD, false>), dim3(n), dim3(512), 0, s, a);
  } else {
    if (a.qhead)
      hipLaunchKernelGGL((bwd_dkdv_wide_kernel<E, HD, HDP, true>), dim3(n), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_wide_kernel<E, HD, HDP, false>), dim3(n), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_wide(int dtype, int hd, const BwdKVArgs &a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool f = dtype == 2;
  switch (hd) {
    case 192: return f ? dkdv_wide<f16, 192, 256>(a, n, s) : dkdv_wide<h16, 192, 256>(a, n, s);
    case 256: return f ? dkdv_wide<f16, 256, 256>(a, n, s) : dkdv_wide<h16, 256, 256>(a, n, s);
    case 512: return f ? dkdv_wide<f16, 512, 512>(a, n, s) : dkdv_wide<h16, 512, 512>(a, n, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dkv
