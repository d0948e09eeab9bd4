// dkv_walks.h -- the index walks of the work items ("DualKV", arXiv 2605.15422, §3.1
// key regions of a query tile, §3.2 the rows a key tile sees): which key tiles a query
// item visits, and in which order a key item visits its query-row steps.  Plain
// integer logic, compiled for the device by the kernels and for the host by the
// work-list check; Cu::load(cu, i) reads sequence bound i (the kernels: ScalarCu, a
// scalar load, defined in dkv_tiles.h).
#pragma once

#include "dkv_launch.h"

namespace dkv {

struct ScalarCu;

__host__ __device__ __forceinline__ int walk_min(int a, int b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ int walk_max(int a, int b) { return a > b ? a : b; }

// The key tiles of a query work item (rows t0 .. t0 + nt - 1 of its sequence, after a
// P-token prompt, window wl or -1): first the prompt tiles its rows can see, then tiles
// of its own keys, BN keys each, at multiples of BN within their region.
template <int BN> struct KeyTiles {
  int ctx_t0, n_ctx, own_t0, n;
  __host__ __device__ __forceinline__ void init(int P, int wl, int t0, int nt) {
    const int ctx_lo = (wl >= 0) ? walk_max(0, P + t0 - wl) : 0;
    ctx_t0 = (ctx_lo / BN) * BN;
    n_ctx = (P > ctx_lo) ? (P - ctx_t0 + BN - 1) / BN : 0;
    const int own_lo = (wl >= 0) ? walk_max(0, t0 - wl) : 0;
    own_t0 = (own_lo / BN) * BN;
    n = n_ctx + (t0 + nt - own_t0 + BN - 1) / BN;
  }
  // Whether tile i lies in the prompt (else in the item's own keys), and its first key
  // within that region.
  __host__ __device__ __forceinline__ bool in_ctx(int i) const { return i < n_ctx; }
  __host__ __device__ __forceinline__ int ctx_start(int i) const { return ctx_t0 + i * BN; }
  __host__ __device__ __forceinline__ int own_start(int i) const { return own_t0 + (i - n_ctx) * BN; }
  // Tile i: the rows of its region from its first key (nrows; rows past them are zero
  // filled) and the logical position of its first key.
  __host__ __device__ __forceinline__ void at(int i, int P, int seqlen, int &nrows, int &kpos0) const {
    if (in_ctx(i)) {
      const int s = ctx_start(i);
      nrows = P - s;
      kpos0 = s;
    } else {
      const int s = own_start(i);
      nrows = seqlen - s;
      kpos0 = P + s;
    }
  }
};

// The query-row steps of a key work item: BM flattened (token, head) rows at a time,
// walked from the item's last sequence and its last step backward, so that every key
// tile of a sequence streams the same rows at the same time (L2 reuse).  A sequence's
// visible rows are [fa, fb) in flattened units: for prompt keys (ctx) all of its rows,
// for its own keys the rows from the tile's first key on, either cut at the window's
// end, and for an item that walks one chunk of them (row_hi > 0) cut to that chunk.
// The cursor keeps the sequence start and length of its seek, so a step's fetch issues
// no scalar load.
//
// Under a window the own keys of a tile see a band of rows as long as the tile plus the
// window, and the bands of neighbouring tiles are shifted by a tile: walked from their
// tops, two tiles that share a row would reach it a tile's worth of steps apart, by
// which time the rows that every tile in flight has read since have pushed it out of
// L2.  A kernel can rotate a windowed own-key walk onto a common clock: with L the
// step count of a whole band (ceil((rot_bn + window_left) G / BM) for tiles of rot_bn
// keys), the walk of a band [sa, sb] of steps starts at the step s* in it with
// s* = 0 (mod L), goes down to sa, then continues from sb down to s* + 1.  Step r of
// every whole band is then visited (s* - r) mod L = -r mod L steps after the item
// starts, the same for every tile, so items that start together read each row at the
// same time and fetch it once.  A band cut short (the sequence's end, a chunk) starts
// at its top when no such s* lies in it.  Every step of the band is visited once
// either way.  The head-dim-split d = 512 dK/dV kernel rotates (on a windowed layer
// its HBM reads drop about sixfold and its time by 4 %); the 128-key kernels walk
// from the top, where the rotation measured 5 % slower.
template <int BM, typename Cu = ScalarCu> struct RowSteps {
  static_assert(kRowChunk % BM == 0, "row chunks follow the step grid");
  const int32_t *cu;
  int seq_lo, key_start, nk_tile, P, wl, G, row_hi, period;
  bool ctx;
  int cs, cf, cfa, cfb, cs0, clen;
  int seg_end;    // the current run of steps ends below this row (a multiple of BM)
  int wrap_row;   // a rotated walk's second run starts at this step row (-1: none)
  int wrap_end;   // and ends below this one
  bool done;
  __host__ __device__ __forceinline__ void seq_range(int sq, int &fa, int &fb, int &s0, int &len) const {
    s0 = Cu::load(cu, sq);
    len = Cu::load(cu, sq + 1) - s0;
    int r_lo, r_hi;
    if (ctx) {
      r_lo = 0;
      r_hi = len;
      if (wl >= 0) r_hi = walk_min(len, key_start + nk_tile - 1 + wl - P + 1);
    } else {
      r_lo = key_start;
      r_hi = len;
      if (wl >= 0) r_hi = walk_min(len, key_start + nk_tile - 1 + wl + 1);
    }
    fa = r_lo * G;
    fb = r_hi > r_lo ? r_hi * G : fa;
    if (row_hi > 0) {
      fa = walk_max(fa, row_hi - kRowChunk);
      fb = walk_max(fa, walk_min(fb, row_hi));
    }
  }
  // From sequence cs downward, the first one with visible rows; its first step.
  __host__ __device__ __forceinline__ void seek() {
    while (cs >= seq_lo) {
      int fa, fb, s0, len;
      seq_range(cs, fa, fb, s0, len);
      if (fb > fa) {
        cfa = fa;
        cfb = fb;
        cs0 = s0;
        clen = len;
        const int sa = fa / BM, sb = (fb - 1) / BM;
        seg_end = sa * BM;
        cf = sb * BM;
        wrap_row = -1;
        if (period > 0) {
          const int s_star = sa + (period - sa % period) % period;
          if (s_star < sb) {
            cf = s_star * BM;
            wrap_row = sb * BM;
            wrap_end = (s_star + 1) * BM;
          }
        }
        return;
      }
      --cs;
    }
    done = true;
  }
  // rot_bn > 0 rotates a windowed own-key walk for key tiles of rot_bn keys (the
  // period is that of a whole tile); 0 walks every band from its top.
  __host__ __device__ __forceinline__ void init(const int32_t *cu_, const KVItem &it, int nk_tile_,
                                       int P_, int wl_, int G_, bool ctx_, int rot_bn) {
    cu = cu_;
    seq_lo = it.seq_lo;
    key_start = it.key_start;
    nk_tile = nk_tile_;
    P = P_;
    wl = wl_;
    G = G_;
    ctx = ctx_;
    row_hi = it.row_hi;
    period = (rot_bn > 0 && wl >= 0 && !ctx) ? ((rot_bn + wl) * G + BM - 1) / BM : 0;
    cs = it.seq_hi - 1;
    cf = cfa = cfb = cs0 = clen = 0;
    done = false;
    seek();
  }
  // The step at the cursor (first row f0, rows [flo, fend) inside the visible range),
  // then the cursor moves on.
  __host__ __device__ __forceinline__ void advance(int &f0, int &flo, int &fend) {
    f0 = cf;
    flo = walk_max(cf, cfa);
    fend = walk_min(cf + BM, cfb);
    cf -= BM;
    if (cf < seg_end) {
      if (wrap_row >= 0) {
        cf = wrap_row;
        seg_end = wrap_end;
        wrap_row = -1;
      } else {
        --cs;
        seek();
      }
    }
  }
};

}  // namespace dkv
