// dkv_launch.h -- host-visible kernel argument blocks and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dkv {

// Key/value tile height of the forward and dQ kernels; query rows per workgroup
// (4 waves x 32 rows).  A workgroup's query rows are bm_tok tokens x G heads of one
// kv head, token-major, so each 32-row wave block mixes tokens and heads.
static constexpr int kFwdBN = 64;
static constexpr int kRowsPerWG = 128;
// Key rows per dK/dV workgroup (4 waves x 32 keys) and query rows per step.
static constexpr int kBwdBN = 128;
static constexpr int kBwdBM = 32;
// Head dims 192, 256, 512 (the head dim is split across the waves of a workgroup):
// query rows per forward workgroup (four pairs of waves), query rows per dQ workgroup
// and keys per dK/dV workgroup (two groups of four waves each), and the largest
// Hq / Hkv they take.
static constexpr int kFwdRowsWide = 128;
static constexpr int kRowsPerWGWide = 64;
static constexpr int kBwdBNWide = 64;
// Head dims 192 and 256 run the backward in pairs of waves: keys per dK/dV workgroup
// and query rows per dQ workgroup (four pairs, 32 each).
static constexpr int kBwdBNPair = 128;
static constexpr int kRowsPerWGPair = 128;
static constexpr int kMaxGWide = 32;

// Work item of the query-parallel kernels (forward, dQ).
struct QItem {
  int32_t g;          // kv head
  int32_t tile;       // query tile index within the sequence
  int32_t seq_start;  // first row of the sequence in the query / own-key tensors
  int32_t seq_len;    // rows of the sequence
  // The sequence's shared prompt: its first row in the prompt key / value tensors and
  // its length P (the logical offset of the sequence's own rows; 0 = no shared region).
  int32_t ctx_start;
  int32_t ctx_len;
  int32_t pad[2];
};

struct FwdArgs {
  const void *q, *k_ctx, *v_ctx, *k_own, *v_own;
  void *o;
  float *lse;
  const QItem *items;
  // GQA head table, or null for the contiguous map: member j of kv head g is q-head
  // qhead[g * G + j] (else g * G + j).
  const int32_t *qhead;
  int Hq, Hkv, G, bm_tok;
  int window_left;    // -1 global
  int lse_ld;         // tokens per LSE row
  float scale;        // softmax scale
};

hipError_t launch_fwd(int dtype, int head_dim, const FwdArgs &a, int n_items, hipStream_t s);
hipError_t launch_fwd_wide(int dtype, int head_dim, const FwdArgs &a, int n_items, hipStream_t s);

// ---- backward ----

// Dneg[h][t] = -sum_c dO[t][h][c] * O[t][h][c] (fp32), rows = T tokens x Hq heads; also
// lsn[h][t] = -LSE[h][t] / scale, the row's log-sum-exp in units of the raw dot product
// <q, k>, negated.  The key-parallel bf16 kernels start their score and dP accumulators
// from these two, so p = exp2(scale * log2(e) * acc) and dS = p * acc' need no per-element
// subtraction.  This launch serves the fp32 path (dtype 1); in bf16 the dQ kernel writes
// both for its rows (BwdQArgs::Dneg_out / lsn_out).
hipError_t launch_bwd_pre(int dtype, int head_dim, const void *o, const void *dout,
                          const float *lse, float *Dneg, float *lsn, long T, int Hq, float scale,
                          hipStream_t s);
hipError_t launch_fill_zero(float *p, long n, hipStream_t s);
// acc[i] += slices[0][i] + slices[1][i] + ... + slices[n_slices - 1][i], added in
// slice order (the fixed-order reduction of the split mode), slices `stride` apart.
hipError_t launch_split_reduce(float *acc, const float *slices, int n_slices, long stride,
                               long n, hipStream_t s);
// dst[i] = round(src[i]) in dtype (a copy for fp32).
hipError_t launch_cast(int dtype, const float *src, void *dst, long n, hipStream_t s);

struct BwdQArgs {
  const void *q, *k_ctx, *v_ctx, *k_own, *v_own, *dout;
  const float *lse, *Dneg;     // Dneg = -rowsum(dO * O) (fp32: from the preprocess kernel)
  // bf16 (no preprocess launch): the dQ kernel forms D from O and dO itself and writes
  // -D and -LSE / scale of its rows here, for the dK/dV kernel.
  const void *o;
  float *Dneg_out, *lsn_out;
  void *dq;
  const QItem *items;
  const int32_t *qhead;        // GQA head table (as FwdArgs::qhead)
  int Hq, Hkv, G, bm_tok, window_left, lse_ld;
  float scale;
};
hipError_t launch_bwd_dq(int dtype, int head_dim, const BwdQArgs &a, int n_items, hipStream_t s);
hipError_t launch_bwd_dq_wide(int dtype, int head_dim, const BwdQArgs &a, int n_items, hipStream_t s);

// Work item of the key-parallel dK/dV kernel: one key tile of one region of one kv
// head, against the query rows of sequences [seq_lo, seq_hi) (all of one prompt group).
enum { kRegionCtx = 0, kRegionOwn = 1 };
struct KVItem {
  int32_t g;
  int32_t region;     // kRegionCtx: keys of the shared prompt; kRegionOwn: of seq_lo
  int32_t key_start;  // first key of the tile within its region
  int32_t seq_lo, seq_hi;
  // The shared prompt of sequences [seq_lo, seq_hi): its first row in the prompt key /
  // value tensors (and the accumulator) and its length P.
  int32_t ctx_start;
  int32_t ctx_len;
  // 0: the item walks every query row that sees its keys.  Otherwise the item walks
  // only flattened rows [row_hi - kRowChunk, row_hi) of its sequence: one chunk of a
  // key tile whose rows are split over several items, each adding its partial sums
  // into the fp32 accumulator (own-region keys of a call that accumulates).
  int32_t row_hi;
};
// Flattened (token, head) query rows per chunk of a split key tile: a multiple of every
// dK/dV kernel's row step, so chunks follow the step grid.
static constexpr int kRowChunk = 4096;

struct BwdKVArgs {
  const void *q, *dout, *k_ctx, *v_ctx, *k_own, *v_own;
  const float *lse, *Dneg;     // Dneg = -rowsum(dO * O) (written by the dQ kernel, or by
  const float *lsn;            // the preprocess kernel in fp32); lsn = -LSE / scale
  const int32_t *cu;           // prefix sums of the query sequences (the workspace's copy)
  const int32_t *qhead;        // GQA head table (as FwdArgs::qhead)
  void *dk_own, *dv_own;       // direct outputs of own-region keys
  float *acc_dk, *acc_dv;      // fp32 accumulators: ctx-region keys, and own keys if own_to_acc
  // Split mode (non-null split_dk): ctx-region items store their partial sums into
  // slice seq_lo / split_chunk of [slices][prompt rows][Hkv][d] instead of adding
  // atomically.
  float *split_dk, *split_dv;
  long split_stride;           // elements per slice (prompt rows * Hkv * d)
  int split_chunk;             // sequences per ctx item
  const KVItem *items;
  int Hq, Hkv, G, window_left, lse_ld;
  int own_to_acc;
  float scale;
};
hipError_t launch_bwd_dkdv(int dtype, int head_dim, const BwdKVArgs &a, int n_items,
                           hipStream_t s);
hipError_t launch_bwd_dkdv_wide(int dtype, int head_dim, const BwdKVArgs &a, int n_items,
                                hipStream_t s);

// ---- layout conversions (N-copy <-> single-prompt packing, first-token rows) ----

// nrows rows written to each of ndst destination ranges: with t = tab + tab_off, row r
// of the range starting at output row t[nsrc + k] (k < ndst) is the sum over s < nsrc
// of input row t[s] + r (fp32 accumulation, rounded once); nsrc == 1 is a copy (read
// once, written ndst times), nsrc == 0 writes zeros.
struct RowItem {
  int32_t tab_off, nrows, nsrc, ndst;
};
static constexpr int kRowsPerItem = 16;
// row_vecs = 16-byte vectors per row.
hipError_t launch_row_sum(int dtype, const void *in, void *out, const RowItem *items, int n_items,
                          const int32_t *tab, int row_vecs, hipStream_t s);

}  // namespace dkv
