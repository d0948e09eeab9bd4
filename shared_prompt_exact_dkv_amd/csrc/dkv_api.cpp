// dkv_api.cpp -- the C ABI of libdkv (include/dkv.h): argument validation, tile
// scheduling and kernel launches.  No device memory is allocated here; scratch
// lives in the caller's workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dkv.h"
#include "dkv_internal.h"
#include "dkv_launch.h"

using namespace dkv;

namespace {

thread_local std::string g_err;

dkv_status fail(dkv_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dkv_status hip_fail(hipError_t e, const char *what) {
  return fail(DKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int dtype) { return dtype == DKV_FP32 ? 4 : 2; }

// Head dims: 64, 96 and 128 run the kernels in which a wave holds whole rows (96 staged
// in 128-wide rows); 192, 256 and 512 the kernels that split the head dim across waves
// (192 staged in 256-wide rows).
bool is_wide(int d) { return d == 192 || d == 256 || d == 512; }
bool is_head_dim(int d) { return d == 64 || d == 96 || d == 128 || is_wide(d); }

// bf16 and fp16 run the same 16-bit MFMA kernels.
bool is16(int dtype) { return dtype == DKV_BF16 || dtype == DKV_FP16; }
bool known_dtype(int dtype) { return is16(dtype) || dtype == DKV_FP32; }

// ---------------------------------------------------------------- validation --

struct Shape {
  int N, P, Hq, Hkv, G, d, wl, dtype;
  float scale;
  long T;                   // cu[N]
  std::vector<int> cu;
  // Prompt groups: group j's prompt is rows [gctx[j], gctx[j + 1]) of the prompt
  // tensors (and of the shared accumulator) and serves sequences [gseq[j], gseq[j + 1]).
  // A call without groups has one, of all P rows and all N sequences.
  std::vector<int> gctx, gseq;
  std::vector<int> sctx0, sP;  // per sequence: first row and length of its prompt
  // Explicit GQA head map (dkv_params::kv_head_of_q): qhead[g * G + j] is the j-th
  // q-head (in increasing order) of kv head g.  Empty for the contiguous map
  // h = g * G + j, which the kernels compute themselves.
  std::vector<int32_t> qhead;
  int bm_tok;               // query tokens per forward workgroup
  int bm_tok_dq;            // query tokens per dQ workgroup
  int kv_tile;              // keys per dK/dV workgroup
};

// Sequences and prompt groups: cu_seqlens, and the group arrays (dkv_fwd / dkv_bwd
// and the layout conversions).  Fills N, P, T, cu and the per-group / per-sequence
// prompt rows.
dkv_status check_seqs(const dkv_params *p, bool is_ctx, Shape *s) {
  if (!p->cu_seqlens_host) return fail(DKV_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
  s->N = p->num_seqs;
  s->P = p->ctx_len;
  s->cu.assign(p->cu_seqlens_host, p->cu_seqlens_host + p->num_seqs + 1);
  if (s->cu[0] != 0) return fail(DKV_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", s->cu[0]);
  for (int i = 0; i < s->N; ++i)
    if (s->cu[i + 1] < s->cu[i])
      return fail(DKV_ERR_INVALID_ARG, "cu_seqlens decreases at %d (%d -> %d)", i, s->cu[i],
                  s->cu[i + 1]);
  s->T = s->cu[s->N];
  {
    const int ng = p->num_groups;
    if (ng < 0) return fail(DKV_ERR_INVALID_ARG, "num_groups < 0 (%d)", ng);
    if (is_ctx && ng != 0)
      return fail(DKV_ERR_INVALID_ARG, "num_groups must be 0 for dkv_ctx_* calls (got %d)", ng);
    if (ng == 0) {
      s->gctx = {0, s->P};
      s->gseq = {0, s->N};
    } else {
      if (!p->ctx_cu_host || !p->group_seq_cu_host)
        return fail(DKV_ERR_INVALID_ARG, "num_groups = %d needs ctx_cu_host and group_seq_cu_host", ng);
      s->gctx.assign(p->ctx_cu_host, p->ctx_cu_host + ng + 1);
      s->gseq.assign(p->group_seq_cu_host, p->group_seq_cu_host + ng + 1);
      if (s->gctx[0] != 0 || s->gseq[0] != 0)
        return fail(DKV_ERR_INVALID_ARG, "ctx_cu_host[0] and group_seq_cu_host[0] must be 0");
      for (int j = 0; j < ng; ++j) {
        if (s->gctx[j + 1] < s->gctx[j])
          return fail(DKV_ERR_INVALID_ARG, "ctx_cu_host decreases at %d (%d -> %d)", j,
                      s->gctx[j], s->gctx[j + 1]);
        if (s->gseq[j + 1] < s->gseq[j])
          return fail(DKV_ERR_INVALID_ARG, "group_seq_cu_host decreases at %d (%d -> %d)", j,
                      s->gseq[j], s->gseq[j + 1]);
      }
      if (s->gctx[ng] != s->P)
        return fail(DKV_ERR_INVALID_ARG, "ctx_cu_host[num_groups] = %d, ctx_len = %d",
                    s->gctx[ng], s->P);
      if (s->gseq[ng] != s->N)
        return fail(DKV_ERR_INVALID_ARG, "group_seq_cu_host[num_groups] = %d, num_seqs = %d",
                    s->gseq[ng], s->N);
    }
    s->sctx0.assign(s->N, 0);
    s->sP.assign(s->N, 0);
    for (size_t j = 0; j + 1 < s->gseq.size(); ++j)
      for (int i = s->gseq[j]; i < s->gseq[j + 1]; ++i) {
        s->sctx0[i] = s->gctx[j];
        s->sP[i] = s->gctx[j + 1] - s->gctx[j];
      }
  }
  return DKV_OK;
}

dkv_status check_params(const dkv_params *p, bool is_ctx, Shape *s) {
  if (!p) return fail(DKV_ERR_INVALID_ARG, "params is NULL");
  if (p->num_seqs < 0) return fail(DKV_ERR_INVALID_ARG, "num_seqs < 0 (%d)", p->num_seqs);
  if (p->ctx_len < 0) return fail(DKV_ERR_INVALID_ARG, "ctx_len < 0 (%d)", p->ctx_len);
  if (is_ctx && p->ctx_len != 0)
    return fail(DKV_ERR_INVALID_ARG, "ctx_len must be 0 for dkv_ctx_* calls (got %d)", p->ctx_len);
  if (p->num_heads_q <= 0 || p->num_heads_kv <= 0)
    return fail(DKV_ERR_INVALID_ARG, "head counts must be positive (Hq=%d, Hkv=%d)",
                p->num_heads_q, p->num_heads_kv);
  if (p->num_heads_q % p->num_heads_kv != 0)
    return fail(DKV_ERR_INVALID_ARG, "Hq (%d) is not a multiple of Hkv (%d)", p->num_heads_q,
                p->num_heads_kv);
  if (!is_head_dim(p->head_dim))
    return fail(DKV_ERR_INVALID_ARG, "head_dim must be 64, 96, 128, 192, 256 or 512 (got %d)",
                p->head_dim);
  if (p->window_left < -1)
    return fail(DKV_ERR_INVALID_ARG, "window_left must be -1 or >= 0 (got %d)", p->window_left);
  if (!known_dtype(p->dtype))
    return fail(DKV_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (!(std::isfinite(p->softmax_scale)))
    return fail(DKV_ERR_INVALID_ARG, "softmax_scale is not finite");
  const int G = p->num_heads_q / p->num_heads_kv;
  if (G > kRowsPerWG)
    return fail(DKV_ERR_UNSUPPORTED, "Hq/Hkv = %d exceeds %d", G, kRowsPerWG);
  s->Hq = p->num_heads_q;
  s->Hkv = p->num_heads_kv;
  s->G = G;
  s->d = p->head_dim;
  s->wl = p->window_left;
  s->dtype = p->dtype;
  s->scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
  if (dkv_status st = check_seqs(p, is_ctx, s)) return st;
  s->qhead.clear();
  if (p->kv_head_of_q) {
    // Every kv head must serve exactly G q-heads; the kernels take the members of a kv
    // head in increasing q-head order.  The contiguous map is run as no map.
    std::vector<int> cnt(s->Hkv, 0);
    bool contiguous = true;
    for (int h = 0; h < s->Hq; ++h) {
      const int k = p->kv_head_of_q[h];
      if (k < 0 || k >= s->Hkv)
        return fail(DKV_ERR_INVALID_ARG, "kv_head_of_q[%d] = %d is outside [0, %d)", h, k, s->Hkv);
      ++cnt[k];
      contiguous = contiguous && k == h / G;
    }
    for (int k = 0; k < s->Hkv; ++k)
      if (cnt[k] != G)
        return fail(DKV_ERR_INVALID_ARG,
                    "kv_head_of_q gives kv head %d %d q-heads; every kv head needs Hq / Hkv = %d",
                    k, cnt[k], G);
    if (!contiguous) {
      s->qhead.assign((size_t)s->Hq, 0);
      std::vector<int> fill(s->Hkv, 0);
      for (int h = 0; h < s->Hq; ++h) {
        const int k = p->kv_head_of_q[h];
        s->qhead[(size_t)k * G + fill[k]++] = h;
      }
    }
  }
  {
    // A window at least as long as the longest logical position sees every earlier
    // key: it is the global causal mask, and is run as one (the kernels form key + wl
    // and (key + wl) * G in 32-bit arithmetic).
    long max_pos = 0;
    for (int i = 0; i < s->N; ++i)
      max_pos = std::max<long>(max_pos, (long)s->sP[i] + s->cu[i + 1] - s->cu[i]);
    if (s->wl >= 0 && (long)s->wl >= max_pos) s->wl = -1;
  }
  if (is16(s->dtype)) {
    // The 16-bit backward addresses a sequence's query rows, and the LSE / D rows, with
    // 32-bit byte offsets from the sequence's start (buffer loads): the query rows of
    // one sequence (plus one 64-row step of slack) and Hq * T LSE entries must stay
    // below 2^31 bytes.
    long max_len = 0;
    for (int i = 0; i < s->N; ++i) max_len = std::max<long>(max_len, s->cu[i + 1] - s->cu[i]);
    const long row_bytes = (long)s->Hq * s->d * 2;
    if ((max_len + 64) * row_bytes > 0x7fffffffL)
      return fail(DKV_ERR_UNSUPPORTED,
                  "a sequence of %ld query rows x %ld bytes exceeds the 2^31-byte range of "
                  "the bf16 kernels' offsets", max_len, row_bytes);
    if ((long)s->Hq * s->T * 4 > 0x7fffffffL)
      return fail(DKV_ERR_UNSUPPORTED, "Hq * tokens = %ld LSE entries exceed 2^29",
                  (long)s->Hq * s->T);
  }
  s->bm_tok = kRowsPerWG / G;
  s->bm_tok_dq = s->bm_tok;
  s->kv_tile = kBwdBN;
  if (is_wide(s->d)) {
    // Head dims 192, 256 and 512 split the head dim across the waves of a workgroup:
    // 128 query rows per forward workgroup; at 512, 64 query rows per dQ and 64 keys per
    // dK/dV workgroup, at 192 / 256 (pairs of waves) 128 of each; 16-bit element types
    // only.
    if (!is16(s->dtype))
      return fail(DKV_ERR_UNSUPPORTED, "head_dim %d is implemented for bf16 / fp16 only", s->d);
    if (G > kMaxGWide)
      return fail(DKV_ERR_UNSUPPORTED, "Hq/Hkv = %d exceeds %d at head_dim %d", G, kMaxGWide, s->d);
    s->bm_tok = kFwdRowsWide / G;
    s->bm_tok_dq = (s->d == 512 ? kRowsPerWGWide : kRowsPerWGPair) / G;
    s->kv_tile = s->d == 512 ? kBwdBNWide : kBwdBNPair;
  }
  return DKV_OK;
}

dkv_status check_ptr(const void *ptr, const char *name, bool needed) {
  if (!needed) return DKV_OK;
  if (!ptr) return fail(DKV_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(DKV_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return DKV_OK;
}

// ---------------------------------------------------------------- scheduling --
//
// MI355X dispatches workgroup b of a launch to XCD b % 8, and each XCD has its own
// L2.  The work lists are therefore built per XCD and interleaved: XCD x serves the
// kv heads g with g % 8 == x (a head with fewer than 8 heads in total is spread over
// 8 / Hkv XCDs, by sequence).  On each XCD the items of one (kv head, sequence)
// group run together, so that the group's keys and values (forward, dQ) or query
// rows (dK/dV) are fetched from HBM once and re-read from L2.  Groups are taken
// longest first and, inside a group, items longest first (the visible key range of
// a query tile grows with its index under the causal mask), so the end of the grid
// fills with short items.

constexpr int kXcds = 8;

// The XCD that serves part `part` (a sequence group, or a tile) of kv head g: a head
// owns XCDs g, g + Hkv, ... when Hkv divides 8, else XCD g % 8.
struct HeadXcds {
  int Hkv, span;
  explicit HeadXcds(int hkv) : Hkv(hkv), span((hkv < kXcds && kXcds % hkv == 0) ? kXcds / hkv : 1) {}
  int xcd(int g, int part) const { return (g + (part % span) * Hkv) % kXcds; }
};

template <typename Item>
std::vector<Item> interleave_xcds(std::vector<std::vector<Item>> &lists) {
  size_t total = 0, longest = 0;
  for (auto &l : lists) {
    total += l.size();
    longest = std::max(longest, l.size());
  }
  std::vector<Item> out;
  out.reserve(total);
  for (size_t k = 0; k < longest; ++k)
    for (auto &l : lists)
      if (k < l.size()) out.push_back(l[k]);
  return out;
}

long q_item_work(const Shape &s, int bm_tok, int tile, int seqlen, int P, int BN) {
  long t0 = (long)tile * bm_tok;
  long t1 = std::min<long>(seqlen, t0 + bm_tok);
  long qmin = P + t0, qmax = P + t1 - 1;
  long lo = (s.wl >= 0) ? std::max<long>(0, qmin - s.wl) : 0;
  long keys = qmax + 1 - lo;
  return (keys + BN - 1) / BN;
}

std::vector<QItem> build_q_items(const Shape &s, int bm_tok, int BN) {
  struct Rec { long work; int tile; };
  struct Group { long work; int seq; std::vector<Rec> recs; };
  std::vector<Group> groups;
  for (int i = 0; i < s.N; ++i) {
    int len = s.cu[i + 1] - s.cu[i];
    int nt = (len + bm_tok - 1) / bm_tok;
    if (nt == 0) continue;
    Group gr{0, i, {}};
    for (int m = 0; m < nt; ++m) {
      long w = q_item_work(s, bm_tok, m, len, s.sP[i], BN);
      gr.recs.push_back({w, m});
      gr.work += w;
    }
    std::stable_sort(gr.recs.begin(), gr.recs.end(),
                     [](const Rec &a, const Rec &b) { return a.work > b.work; });
    groups.push_back(std::move(gr));
  }
  std::stable_sort(groups.begin(), groups.end(),
                   [](const Group &a, const Group &b) { return a.work > b.work; });
  HeadXcds hx(s.Hkv);
  std::vector<std::vector<QItem>> lists(kXcds);
  // One sequence alone (Call 1) is spread over a head's XCDs tile by tile.
  const bool by_tile = groups.size() < (size_t)hx.span;
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const Group &gr = groups[gi];
    const int start = s.cu[gr.seq], len = s.cu[gr.seq + 1] - start;
    for (int g = 0; g < s.Hkv; ++g)
      for (size_t r = 0; r < gr.recs.size(); ++r)
        lists[hx.xcd(g, (int)(by_tile ? r : gi))].push_back(
            {g, gr.recs[r].tile, start, len, s.sctx0[gr.seq], s.sP[gr.seq], {0, 0}});
  }
  return interleave_xcds(lists);
}

// ------------------------------------------------------- staging of lists --
//
// Work lists and the per-call tables (sequence bounds, head map) are built on the host
// and copied into the workspace on the caller's stream, in one copy per call.
//   Pinned (the entry points with a caller workspace): the copy reads a pinned host
//   slot.  Outside graph capture a slot is reused only once the event recorded after
//   its copy has completed.  Slots are polled, never waited for: when every slot is
//   still in flight a new one is added, so a call never blocks the host (the pool grows
//   with the caller's run-ahead).  Under HIP graph capture the copy becomes a node of
//   the graph, which reads the slot again at every replay, so the slot is reserved for
//   that graph and no later call writes it; it stays reserved until the process ends
//   (a call's staged bytes: 32 per work item plus the sequence and head tables).
//   Slots are never freed while the process runs: freeing pinned memory may wait for
//   the device.
//   Pageable (the entry point that allocates nothing): the copy reads the host vector
//   itself; HIP performs a copy from unpinned host memory synchronously, so the call
//   returns once the data has left the host buffer, which is then free to go.  Such a
//   copy cannot be captured into a graph, so this path refuses a capturing stream.

enum class Staging { kPinned, kPageable };

struct StagingRing {
  struct Slot {
    void *host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;    // an eager copy from it may still be running
    bool captured = false;   // a captured graph reads it at every replay
  };
  std::mutex mu;
  std::map<int, std::vector<Slot>> per_device;
};

// Never destroyed: slots reserved by graphs must outlive every replay.
StagingRing &ring() {
  static StagingRing *r = new StagingRing;
  return *r;
}

// Whether `stream` is capturing a graph.  A capture that an earlier error invalidated
// is reported as an error; with pageable staging an active capture is refused too.
// Runs before anything is enqueued.
dkv_status capture_state(hipStream_t stream, Staging how, bool *capturing) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs == hipStreamCaptureStatusInvalidated)
    return fail(DKV_ERR_HIP, "the stream's graph capture has been invalidated");
  *capturing = cs == hipStreamCaptureStatusActive;
  if (*capturing && how == Staging::kPageable)
    return fail(DKV_ERR_UNSUPPORTED, "calls without a workspace cannot run on a capturing "
                "stream (their work lists are copied from pageable host memory)");
  return DKV_OK;
}

dkv_status upload(const void *src, size_t bytes, void *dst, hipStream_t stream,
                  Staging how = Staging::kPinned) {
  if (bytes == 0) return DKV_OK;
  bool capturing = false;
  dkv_status st = capture_state(stream, how, &capturing);
  if (st != DKV_OK) return st;
  hipError_t e;
  if (how == Staging::kPageable) {
    e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work lists, pageable)");
    return DKV_OK;
  }
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  StagingRing &r = ring();
  std::lock_guard<std::mutex> lock(r.mu);
  auto &slots = r.per_device[dev];
  StagingRing::Slot *fit = nullptr;
  for (auto &x : slots) {
    if (x.captured) continue;
    // Under capture the events are not polled (a slot still pending stays skipped).
    if (x.pending && !capturing) {
      e = hipEventQuery(x.ev);
      if (e == hipSuccess)
        x.pending = false;
      else if (e != hipErrorNotReady)
        return hip_fail(e, "hipEventQuery(staging)");
    }
    if (x.pending) continue;
    if (x.cap >= bytes && (!fit || x.cap < fit->cap)) fit = &x;
  }
  StagingRing::Slot *sl = fit;
  if (!sl) {
    // A new slot (a smaller idle one is kept for smaller lists).  Allocating pinned
    // memory is not a stream operation; the thread's capture mode is relaxed around it
    // so that a capture in global mode accepts the call.
    StagingRing::Slot fresh;
    const size_t cap = std::max<size_t>(bytes, 64 * 1024);
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    if (capturing) (void)hipThreadExchangeStreamCaptureMode(&mode);
    e = hipHostMalloc(&fresh.host, cap, hipHostMallocDefault);
    if (capturing) (void)hipThreadExchangeStreamCaptureMode(&mode);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(staging)");
    fresh.cap = cap;
    slots.push_back(fresh);
    sl = &slots.back();
  }
  std::memcpy(sl->host, src, bytes);
  e = hipMemcpyAsync(dst, sl->host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work lists)");
  if (capturing) {
    sl->captured = true;
    return DKV_OK;
  }
  if (!sl->ev) {
    e = hipEventCreateWithFlags(&sl->ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  e = hipEventRecord(sl->ev, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(staging)");
  sl->pending = true;
  return DKV_OK;
}

// The host image of a call's staged region (work lists and tables at the offsets of the
// workspace plan), copied to the workspace in one upload.
struct StagedImage {
  std::vector<char> bytes;
  explicit StagedImage(size_t n) : bytes(n, 0) {}
  void put(size_t off, const void *src, size_t n) {
    if (n) std::memcpy(bytes.data() + off, src, n);
  }
};

// -------------------------------------------------------------- kernel timing --

enum KernelClass { kKFwd = 0, kKPre, kKDq, kKDkdv, kKZero, kKCast, kKReduce, kKLayout, kKClasses };
const char *const kKernelNames[kKClasses] = {"attn_fwd", "bwd_pre",  "bwd_dq",       "bwd_dkdv",
                                             "acc_zero", "acc_cast", "split_reduce", "layout"};

struct Timing {
  std::mutex mu;
  bool on = false;
  struct Rec { int cls; hipEvent_t a, b; };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
};

Timing &timing() {
  static Timing t;
  return t;
}

hipEvent_t get_event(Timing &t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch `fn` (returning hipError_t) on `stream`, bracketed by events when enabled.
template <typename F> hipError_t timed(int cls, hipStream_t stream, F &&fn) {
  Timing &t = timing();
  if (!t.on) return fn();
  // A capturing stream records no timing events (they would become nodes of the graph).
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return fn();
  std::lock_guard<std::mutex> lock(t.mu);
  hipEvent_t a = get_event(t), b = get_event(t);
  if (!a || !b) return fn();
  hipEventRecord(a, stream);
  hipError_t e = fn();
  hipEventRecord(b, stream);
  t.recs.push_back({cls, a, b});
  return e;
}

// ------------------------------------------------------------ workspace plans --

// A call's staged region: its work lists, then the tables the kernels read (the host
// copy of cu_seqlens for the key-parallel kernels, the GQA head table when a map is
// given), at 256-byte aligned offsets from the region's start.
struct StagedPlan {
  size_t q_off = 0, kv_off = 0, cu_off = 0, qhead_off = 0, bytes = 0;
  size_t n_q = 0, n_kv = 0;
};

StagedPlan plan_staged(const Shape &s, size_t n_q, size_t n_kv, bool with_cu) {
  StagedPlan sp;
  sp.n_q = n_q;
  sp.n_kv = n_kv;
  sp.q_off = 0;
  sp.kv_off = sp.q_off + align_up(n_q * sizeof(QItem));
  sp.cu_off = sp.kv_off + align_up(n_kv * sizeof(KVItem));
  sp.qhead_off = sp.cu_off + (with_cu ? align_up((size_t)(s.N + 1) * sizeof(int32_t)) : 0);
  sp.bytes = sp.qhead_off + align_up(s.qhead.size() * sizeof(int32_t));
  return sp;
}

struct FwdPlan {
  StagedPlan st;   // at offset 0 of the workspace
  size_t bytes = 0;
};

size_t count_q_items(const Shape &s, int bm_tok) {
  size_t n = 0;
  for (int i = 0; i < s.N; ++i) {
    int len = s.cu[i + 1] - s.cu[i];
    n += (size_t)((len + bm_tok - 1) / bm_tok) * s.Hkv;
  }
  return n;
}

FwdPlan plan_fwd(const Shape &s) {
  FwdPlan pl;
  pl.st = plan_staged(s, count_q_items(s, s.bm_tok), 0, false);
  pl.bytes = pl.st.n_q ? pl.st.bytes : 0;
  return pl;
}

dkv_status check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return DKV_OK;
  if (!ws) return fail(DKV_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(DKV_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(DKV_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return DKV_OK;
}

const int32_t *qhead_dev(const Shape &s, char *staged, const StagedPlan &sp) {
  return s.qhead.empty() ? nullptr : reinterpret_cast<const int32_t *>(staged + sp.qhead_off);
}

dkv_status run_fwd(const Shape &s, const void *q, const void *kc, const void *vc,
                   const void *ko, const void *vo, void *o, float *lse, void *ws,
                   size_t ws_bytes, hipStream_t stream, Staging how) {
  FwdPlan pl = plan_fwd(s);
  dkv_status st = check_ws(ws, ws_bytes, pl.bytes);
  if (st != DKV_OK) return st;
  bool capturing = false;
  if (pl.st.n_q > 0 && (st = capture_state(stream, how, &capturing)) != DKV_OK) return st;
  if (pl.st.n_q == 0) return DKV_OK;
  std::vector<QItem> items = build_q_items(s, s.bm_tok, kFwdBN);
  char *wsb = static_cast<char *>(ws);
  StagedImage img(pl.st.bytes);
  img.put(pl.st.q_off, items.data(), items.size() * sizeof(QItem));
  img.put(pl.st.qhead_off, s.qhead.data(), s.qhead.size() * sizeof(int32_t));
  st = upload(img.bytes.data(), img.bytes.size(), wsb, stream, how);
  if (st != DKV_OK) return st;
  FwdArgs a{};
  a.q = q;
  a.k_ctx = kc;
  a.v_ctx = vc;
  a.k_own = ko;
  a.v_own = vo;
  a.o = o;
  a.lse = lse;
  a.items = reinterpret_cast<const QItem *>(wsb + pl.st.q_off);
  a.qhead = qhead_dev(s, wsb, pl.st);
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.bm_tok = s.bm_tok;
  a.window_left = s.wl;
  a.lse_ld = (int)s.T;
  a.scale = s.scale;
  hipError_t e = timed(kKFwd, stream, [&] { return launch_fwd(s.dtype, s.d, a, (int)items.size(), stream); });
  if (e != hipSuccess) return hip_fail(e, "fwd kernel launch");
  return DKV_OK;
}

// Key-parallel work items (dK/dV): one per (kv head, key tile) of each sequence's own
// keys, and per (kv head, prompt key tile, chunk of sequences) of the shared prompt.
// The chunk size sets how many sequences' partial dK_P/dV_P a workgroup sums in
// registers before one atomic add per element.  Global layers: 4 (fewer sequences when
// N < 4), which quarters the accumulator's atomic traffic and measured 0.2-2.2 % faster
// per step than 1 on every global workload benchmarked; 8 was no better at d = 128 and
// 27 % slower on the d = 512 global layer (N = 8: one chunk, too few and too long
// items).  Windowed layers: 1.  There the responses see only the prompt's last window
// of keys, so those items are few and short, and grouped by four they finish the launch
// as a tail of long items (d = 256 and 512 windowed steps 4-6 % slower).  DKV_CTX_CHUNK
// overrides it (tuning only).

int ctx_chunk(const Shape &s) {
  static int env = [] {
    const char *e = getenv("DKV_CTX_CHUNK");
    return e ? atoi(e) : 0;
  }();
  const int c = env > 0 ? env : (s.wl >= 0 ? 1 : 4);
  return std::min(c, std::max(1, s.N));
}

// Split mode: the prompt-key terms of the N responses go to S slices, one per chunk
// of ceil(N / S) sequences summed in registers; S = min(N, 8) unless DKV_SPLIT_SLICES
// sets it.  Returns the chunk size; the slice count is ceil(N / chunk).
int split_chunk(const Shape &s) {
  static int env = [] {
    const char *e = getenv("DKV_SPLIT_SLICES");
    return e ? atoi(e) : 0;
  }();
  const int n = std::max(1, s.N);
  const int slices = std::min(n, env > 0 ? env : 8);
  return (n + slices - 1) / slices;
}
int split_slices(const Shape &s) {
  const int cs = split_chunk(s);
  return (std::max(1, s.N) + cs - 1) / cs;
}

long kv_rows_visible(const Shape &s, bool ctx, int key_start, int nk, int len, int P) {
  long lo, hi;
  if (ctx) {
    lo = 0;
    hi = len;
    if (s.wl >= 0) hi = std::min<long>(len, (long)key_start + nk - 1 + s.wl - P + 1);
  } else {
    lo = key_start;
    hi = len;
    if (s.wl >= 0) hi = std::min<long>(len, (long)key_start + nk - 1 + s.wl + 1);
  }
  return std::max<long>(0, hi - lo);
}

// Own-region key tiles of a call that adds them into the accumulator may be split into
// row chunks (see KVItem::row_hi): when the call's key tiles alone would give fewer
// workgroups than this (two per slot of the GPU's 256 CUs x 2 resident workgroups), the
// causal walk's long first tiles leave most of the GPU idle.  With more, the tiles
// already fill the GPU and chunks would only add accumulator traffic.
static constexpr long kChunkBelowItems = 1024;

bool chunk_own_rows(const Shape &s) {
  long tiles = 0;
  for (int i = 0; i < s.N; ++i) tiles += (s.cu[i + 1] - s.cu[i] + s.kv_tile - 1) / s.kv_tile;
  return tiles * s.Hkv < kChunkBelowItems;
}

// The work items of an own-region key tile (keys k0 .. k0 + nk - 1 of a sequence of len
// rows): (row_hi, visible rows) each.  Unsplit, one item walks every row that sees the
// tile (row_hi = 0); split, one item per kRowChunk-row chunk (on multiples of kRowChunk
// flattened rows) of those rows, when they span more than one chunk's worth.
std::vector<std::pair<int, long>> own_row_chunks(const Shape &s, int k0, int nk, int len,
                                                 bool chunk) {
  const long rows = kv_rows_visible(s, false, k0, nk, len, 0);
  const long fa = (long)k0 * s.G, fb = fa + rows * s.G;   // flattened rows [fa, fb)
  std::vector<std::pair<int, long>> out;
  if (!chunk || fb - fa <= kRowChunk) {
    out.push_back({0, rows});
    return out;
  }
  for (long c = fa / kRowChunk; c * kRowChunk < fb; ++c) {
    const long lo = std::max(fa, c * kRowChunk), hi = std::min(fb, (c + 1) * kRowChunk);
    out.push_back({(int)((c + 1) * kRowChunk), (hi - lo + s.G - 1) / s.G});
  }
  return out;
}

// The chunks of sequences [lo, hi) of prompt group pg whose prompt-key tiles are
// separate work items.  Split mode takes the global chunks of split_chunk() sequences
// (chunk c fills slice c), clipped to the group; a chunk holding no sequence of the
// group becomes the empty range [c * chunk, c * chunk), whose items store zeros, so that
// every slice element of the group's prompt rows is written once.  Otherwise chunks of
// ctx_chunk() sequences from the group's first one.
std::vector<std::pair<int, int>> ctx_chunks(const Shape &s, int pg, bool split) {
  std::vector<std::pair<int, int>> out;
  const int q0 = s.gseq[pg], q1 = s.gseq[pg + 1];
  if (split) {
    const int cs = split_chunk(s), n = split_slices(s);
    for (int c = 0; c < n; ++c) {
      int lo = std::max(q0, c * cs), hi = std::min(q1, (c + 1) * cs);
      if (hi <= lo) lo = hi = c * cs;
      out.push_back({lo, hi});
    }
  } else {
    const int cs = ctx_chunk(s);
    for (int lo = q0; lo < q1; lo += cs) out.push_back({lo, std::min(q1, lo + cs)});
  }
  return out;
}

std::vector<KVItem> build_kv_items(const Shape &s, bool with_ctx, bool split,
                                   bool chunk_own = false) {
  // Per prompt group and chunk of its sequences: the prompt key tiles that add the
  // chunk's terms to the shared accumulator, and the chunk's own response key tiles
  // (row chunks of them with chunk_own).  All of them stream the chunk's query rows.
  struct Rec { long work; int region, key_start, lo, hi, c0, Pg, row_hi; };
  struct Group { long work; std::vector<Rec> recs; };
  std::vector<Group> groups;
  auto add = [&](Group &x) {
    if (x.recs.empty()) return;
    for (const Rec &r : x.recs) x.work += r.work;
    std::stable_sort(x.recs.begin(), x.recs.end(),
                     [](const Rec &a, const Rec &b) { return a.work > b.work; });
    groups.push_back(std::move(x));
  };
  for (int pg = 0; pg + 1 < (int)s.gseq.size(); ++pg) {
    const int c0 = s.gctx[pg], Pg = s.gctx[pg + 1] - c0;
    const bool ctx_here = with_ctx && Pg > 0;
    std::vector<std::pair<int, int>> chunks = ctx_chunks(s, pg, split && ctx_here);
    for (const auto &ch : chunks) {
      const int lo = ch.first, hi = ch.second;
      // The chunk's prompt-key tiles and its own-key tiles form separate groups: the
      // prompt-key tiles all walk the same rows (every row of the chunk), so a group of
      // them shares its row blocks in L2.  The own-key tiles of the chunk's sequences
      // form one group, longest first across the sequences: on the Qwen3-8B-shaped step
      // that measured 1.2 % faster than one group per sequence, although the launch then
      // reads twice the bytes (a sequence's tiles are split between two generations of
      // workgroups, so its rows are fetched twice).
      Group ctxg{0, {}}, owng{0, {}};
      if (ctx_here) {
        for (int k0 = 0; k0 < Pg; k0 += s.kv_tile) {
          int nk = std::min(s.kv_tile, Pg - k0);
          long w = 0;
          for (int i = lo; i < hi; ++i)
            w += kv_rows_visible(s, true, k0, nk, s.cu[i + 1] - s.cu[i], Pg);
          // Split mode keeps tiles no row of the chunk sees: they store the zeros of
          // their slice, so every slice element is written.
          if (w > 0 || split) ctxg.recs.push_back({w, kRegionCtx, k0, lo, hi, c0, Pg, 0});
        }
      }
      for (int i = lo; i < hi; ++i) {
        int len = s.cu[i + 1] - s.cu[i];
        for (int k0 = 0; k0 < len; k0 += s.kv_tile) {
          int nk = std::min(s.kv_tile, len - k0);
          for (const auto &ch : own_row_chunks(s, k0, nk, len, chunk_own))
            owng.recs.push_back({ch.second, kRegionOwn, k0, i, i + 1, c0, Pg, ch.first});
        }
      }
      add(ctxg);
      add(owng);
    }
  }
  std::stable_sort(groups.begin(), groups.end(),
                   [](const Group &a, const Group &b) { return a.work > b.work; });
  HeadXcds hx(s.Hkv);
  std::vector<std::vector<KVItem>> lists(kXcds);
  const bool by_tile = groups.size() < (size_t)hx.span;
  for (size_t gi = 0; gi < groups.size(); ++gi)
    for (int g = 0; g < s.Hkv; ++g)
      for (size_t r = 0; r < groups[gi].recs.size(); ++r) {
        const Rec &x = groups[gi].recs[r];
        lists[hx.xcd(g, (int)(by_tile ? r : gi))].push_back(
            {g, x.region, x.key_start, x.lo, x.hi, x.c0, x.Pg, x.row_hi});
      }
  return interleave_xcds(lists);
}

struct BwdPlan {
  size_t d_off = 0, l2_off = 0, st_off = 0, split_off = 0, bytes = 0;
  StagedPlan st;   // at st_off
  int slices = 0;
};

BwdPlan plan_bwd(const Shape &s, bool with_ctx, bool split, bool chunk_own = false) {
  BwdPlan pl;
  size_t nkv = 0;
  for (int i = 0; i < s.N; ++i) {
    int len = s.cu[i + 1] - s.cu[i];
    for (int k0 = 0; k0 < len; k0 += s.kv_tile)
      nkv += own_row_chunks(s, k0, std::min(s.kv_tile, len - k0), len, chunk_own).size();
  }
  if (with_ctx)
    for (int pg = 0; pg + 1 < (int)s.gseq.size(); ++pg) {
      const int Pg = s.gctx[pg + 1] - s.gctx[pg];
      if (Pg > 0)
        nkv += (size_t)((Pg + s.kv_tile - 1) / s.kv_tile) * ctx_chunks(s, pg, split).size();
    }
  // nkv * Hkv is an upper bound (empty windowed items are dropped)
  pl.st = plan_staged(s, count_q_items(s, s.bm_tok_dq), nkv * s.Hkv, true);
  pl.d_off = 0;
  pl.l2_off = align_up((size_t)s.Hq * s.T * sizeof(float));
  pl.st_off = pl.l2_off + align_up((size_t)s.Hq * s.T * sizeof(float));
  pl.split_off = pl.st_off + pl.st.bytes;
  pl.bytes = pl.split_off;
  if (split && with_ctx && s.P > 0) {   // dK and dV slices
    pl.slices = split_slices(s);
    pl.bytes += 2 * align_up((size_t)pl.slices * s.P * s.Hkv * s.d * sizeof(float));
  }
  if (s.T == 0) pl.bytes = 0;
  return pl;
}

struct BwdIO {
  const void *q, *kc, *vc, *ko, *vo, *o, *dout;
  const float *lse;
  void *dq, *dk_own, *dv_own;
  float *acc_dk, *acc_dv;
  long acc_rows;      // rows of the accumulator (P for the shared prompt)
  int flags;
  void *dk_fin, *dv_fin;
  bool with_ctx, own_to_acc;
};

dkv_status run_bwd(const Shape &s, const BwdIO &io, void *ws, size_t ws_bytes,
                   hipStream_t stream, Staging how) {
  const bool split = (io.flags & DKV_ACC_SPLIT) && io.with_ctx && s.P > 0;
  // Own key tiles split into row chunks: a call that adds them into the accumulator
  // (Call 1 with one), unless DKV_ACC_SPLIT asks for one writer per element.
  const bool chunk = io.own_to_acc && !(io.flags & DKV_ACC_SPLIT) && chunk_own_rows(s);
  BwdPlan pl = plan_bwd(s, io.with_ctx, split, chunk);
  dkv_status st = check_ws(ws, ws_bytes, pl.bytes);
  if (st != DKV_OK) return st;
  bool capturing = false;
  if ((st = capture_state(stream, how, &capturing)) != DKV_OK) return st;
  char *wsb = static_cast<char *>(ws);
  const long acc_elems = io.acc_rows * s.Hkv * s.d;
  hipError_t e;
  if ((io.flags & DKV_ACC_ZERO) && io.acc_dk) {
    e = timed(kKZero, stream, [&] {
      hipError_t r = launch_fill_zero(io.acc_dk, acc_elems, stream);
      return r != hipSuccess ? r : launch_fill_zero(io.acc_dv, acc_elems, stream);
    });
    if (e != hipSuccess) return hip_fail(e, "zero acc");
  }
  if (s.T > 0) {
    float *Dneg = reinterpret_cast<float *>(wsb + pl.d_off);
    float *lsn = reinterpret_cast<float *>(wsb + pl.l2_off);
    const bool fused_pre = is16(s.dtype);   // the 16-bit dQ kernels form -D, -LSE/scale
    if (!fused_pre) {
      e = timed(kKPre, stream, [&] {
        return launch_bwd_pre(s.dtype, s.d, io.o, io.dout, io.lse, Dneg, lsn, s.T, s.Hq, s.scale,
                              stream);
      });
      if (e != hipSuccess) return hip_fail(e, "bwd preprocess launch");
    }
    std::vector<QItem> qi = build_q_items(s, s.bm_tok_dq, kFwdBN);
    std::vector<KVItem> kv = build_kv_items(s, io.with_ctx, split, chunk);
    if (qi.size() != pl.st.n_q || kv.size() > pl.st.n_kv)
      return fail(DKV_ERR_INVALID_ARG, "internal: work lists exceed their plan");
    char *stb = wsb + pl.st_off;
    {
      StagedImage img(pl.st.bytes);
      img.put(pl.st.q_off, qi.data(), qi.size() * sizeof(QItem));
      img.put(pl.st.kv_off, kv.data(), kv.size() * sizeof(KVItem));
      img.put(pl.st.cu_off, s.cu.data(), s.cu.size() * sizeof(int32_t));
      img.put(pl.st.qhead_off, s.qhead.data(), s.qhead.size() * sizeof(int32_t));
      if ((st = upload(img.bytes.data(), img.bytes.size(), stb, stream, how)) != DKV_OK) return st;
    }
    BwdQArgs qa{};
    qa.q = io.q; qa.k_ctx = io.kc; qa.v_ctx = io.vc; qa.k_own = io.ko; qa.v_own = io.vo;
    qa.dout = io.dout; qa.lse = io.lse; qa.Dneg = Dneg; qa.dq = io.dq;
    if (fused_pre) {
      qa.o = io.o;
      qa.Dneg_out = Dneg;
      qa.lsn_out = lsn;
    }
    qa.items = reinterpret_cast<const QItem *>(stb + pl.st.q_off);
    qa.qhead = qhead_dev(s, stb, pl.st);
    qa.Hq = s.Hq; qa.Hkv = s.Hkv; qa.G = s.G; qa.bm_tok = s.bm_tok_dq;
    qa.window_left = s.wl; qa.lse_ld = (int)s.T; qa.scale = s.scale;
    e = timed(kKDq, stream, [&] { return launch_bwd_dq(s.dtype, s.d, qa, (int)qi.size(), stream); });
    if (e != hipSuccess) return hip_fail(e, "dq kernel launch");
    BwdKVArgs ka{};
    ka.q = io.q; ka.dout = io.dout; ka.k_ctx = io.kc; ka.v_ctx = io.vc; ka.k_own = io.ko;
    ka.v_own = io.vo; ka.lse = io.lse; ka.Dneg = Dneg; ka.lsn = lsn;
    ka.cu = reinterpret_cast<const int32_t *>(stb + pl.st.cu_off);
    ka.qhead = qa.qhead;
    ka.dk_own = io.dk_own; ka.dv_own = io.dv_own; ka.acc_dk = io.acc_dk; ka.acc_dv = io.acc_dv;
    ka.items = reinterpret_cast<const KVItem *>(stb + pl.st.kv_off);
    ka.Hq = s.Hq; ka.Hkv = s.Hkv; ka.G = s.G; ka.window_left = s.wl;
    ka.lse_ld = (int)s.T; ka.own_to_acc = io.own_to_acc ? 1 : 0;
    ka.scale = s.scale;
    float *slices = reinterpret_cast<float *>(wsb + pl.split_off);
    const long slice_elems = (long)s.P * s.Hkv * s.d;
    const size_t slice_bytes = align_up((size_t)pl.slices * slice_elems * sizeof(float));
    if (split) {
      ka.split_dk = slices;
      ka.split_dv = reinterpret_cast<float *>(wsb + pl.split_off + slice_bytes);
      ka.split_stride = slice_elems;
      ka.split_chunk = split_chunk(s);
    }
    e = timed(kKDkdv, stream, [&] { return launch_bwd_dkdv(s.dtype, s.d, ka, (int)kv.size(), stream); });
    if (e != hipSuccess) return hip_fail(e, "dkdv kernel launch");
    if (split) {
      e = timed(kKReduce, stream, [&] {
        hipError_t r = launch_split_reduce(io.acc_dk, ka.split_dk, pl.slices, slice_elems,
                                           acc_elems, stream);
        return r != hipSuccess ? r
                               : launch_split_reduce(io.acc_dv, ka.split_dv, pl.slices,
                                                     slice_elems, acc_elems, stream);
      });
      if (e != hipSuccess) return hip_fail(e, "split reduce launch");
    }
  }
  if ((io.flags & DKV_ACC_FINALIZE) && io.acc_dk) {
    e = timed(kKCast, stream, [&] {
      hipError_t r = launch_cast(s.dtype, io.acc_dk, io.dk_fin, acc_elems, stream);
      return r != hipSuccess ? r : launch_cast(s.dtype, io.acc_dv, io.dv_fin, acc_elems, stream);
    });
    if (e != hipSuccess) return hip_fail(e, "cast launch");
  }
  return DKV_OK;
}

// ------------------------------------------------------- layout conversions --
//
// Row maps between the N-copy packing (copy i = its prompt's rows then its own rows,
// copies in sequence order) and the single-prompt packing (every prompt once, in group
// order, then every response).  Each segment of consecutive rows becomes work items of
// at most kRowsPerItem rows.

struct LayoutPlan {
  std::vector<RowItem> items;
  std::vector<int32_t> src;   // per item: its source row starts, then its destination starts
  long in_rows = 0, out_rows = 0;
  size_t items_off = 0, src_off = 0, bytes = 0;
};

// n rows written to each output range starting at dsts: the sum over the given input
// row starts (each advanced with the row), a copy for one start, zeros for none.  An
// item of several sources or destinations takes fewer rows, so that it moves about as
// much as a plain copy item.
void add_segment(LayoutPlan &pl, const std::vector<long> &dsts, long n,
                 const std::vector<long> &starts) {
  const long fan = std::max<long>(1, std::max<long>((long)starts.size(), (long)dsts.size()));
  const long rows = std::max<long>(1, kRowsPerItem / fan);
  for (long k = 0; k < n; k += rows) {
    RowItem it;
    it.tab_off = (int32_t)pl.src.size();
    it.nrows = (int32_t)std::min<long>(rows, n - k);
    it.nsrc = (int32_t)starts.size();
    it.ndst = (int32_t)dsts.size();
    for (long st : starts) pl.src.push_back((int32_t)(st + k));
    for (long d : dsts) pl.src.push_back((int32_t)(d + k));
    pl.items.push_back(it);
  }
}
void add_segment(LayoutPlan &pl, long dst, long n, const std::vector<long> &starts) {
  add_segment(pl, std::vector<long>{dst}, n, starts);
}

LayoutPlan plan_layout(const Shape &s, int op) {
  LayoutPlan pl;
  std::vector<long> nc0(s.N + 1, 0);   // first row of each copy in the N-copy packing
  for (int i = 0; i < s.N; ++i) nc0[i + 1] = nc0[i] + s.sP[i] + (s.cu[i + 1] - s.cu[i]);
  const long packed = (long)s.P + s.T;
  const int ngroups = (int)s.gseq.size() - 1;
  auto len = [&](int i) { return (long)(s.cu[i + 1] - s.cu[i]); };
  switch (op) {
    case DKV_PACK:   // N-copy -> single-prompt: prompts from each group's first copy
      pl.in_rows = nc0[s.N];
      pl.out_rows = packed;
      for (int j = 0; j < ngroups; ++j) {
        std::vector<long> st;
        if (s.gseq[j + 1] > s.gseq[j]) st.push_back(nc0[s.gseq[j]]);
        add_segment(pl, s.gctx[j], s.gctx[j + 1] - s.gctx[j], st);
      }
      for (int i = 0; i < s.N; ++i) add_segment(pl, s.P + s.cu[i], len(i), {nc0[i] + s.sP[i]});
      break;
    case DKV_UNPACK:   // single-prompt -> N-copy: each copy takes its group's prompt
      pl.in_rows = packed;
      pl.out_rows = nc0[s.N];
      for (int j = 0; j < ngroups; ++j) {   // a prompt chunk is read once per group
        std::vector<long> dsts;
        for (int i = s.gseq[j]; i < s.gseq[j + 1]; ++i) dsts.push_back(nc0[i]);
        if (!dsts.empty()) add_segment(pl, dsts, s.gctx[j + 1] - s.gctx[j], {(long)s.gctx[j]});
      }
      for (int i = 0; i < s.N; ++i) add_segment(pl, nc0[i] + s.sP[i], len(i), {(long)s.P + s.cu[i]});
      break;
    case DKV_UNPACK_BWD:   // adjoint of UNPACK: a prompt row sums its group's copies
      pl.in_rows = nc0[s.N];
      pl.out_rows = packed;
      for (int j = 0; j < ngroups; ++j) {
        std::vector<long> st;
        for (int i = s.gseq[j]; i < s.gseq[j + 1]; ++i) st.push_back(nc0[i]);
        add_segment(pl, s.gctx[j], s.gctx[j + 1] - s.gctx[j], st);
      }
      for (int i = 0; i < s.N; ++i) add_segment(pl, s.P + s.cu[i], len(i), {nc0[i] + s.sP[i]});
      break;
    case DKV_FIRST_TOKEN_GATHER:   // predictor row of every response token
      pl.in_rows = packed;
      pl.out_rows = s.T;
      for (int i = 0; i < s.N; ++i) {
        if (len(i) == 0) continue;
        std::vector<long> st;
        if (s.sP[i] > 0) st.push_back(s.sctx0[i] + s.sP[i] - 1);   // the last prompt row
        add_segment(pl, s.cu[i], 1, st);
        add_segment(pl, s.cu[i] + 1, len(i) - 1, {(long)s.P + s.cu[i]});
      }
      break;
    case DKV_FIRST_TOKEN_SCATTER:   // adjoint of the gather
      pl.in_rows = s.T;
      pl.out_rows = packed;
      for (int j = 0; j < ngroups; ++j) {
        const long Pg = s.gctx[j + 1] - s.gctx[j];
        if (Pg == 0) continue;
        add_segment(pl, s.gctx[j], Pg - 1, {});
        std::vector<long> st;
        for (int i = s.gseq[j]; i < s.gseq[j + 1]; ++i)
          if (len(i) > 0) st.push_back(s.cu[i]);
        add_segment(pl, s.gctx[j + 1] - 1, 1, st);
      }
      for (int i = 0; i < s.N; ++i) {
        if (len(i) == 0) continue;
        add_segment(pl, s.P + s.cu[i], len(i) - 1, {(long)s.cu[i] + 1});
        add_segment(pl, s.P + s.cu[i] + len(i) - 1, 1, {});
      }
      break;
  }
  pl.items_off = 0;
  pl.src_off = align_up(pl.items.size() * sizeof(RowItem));
  pl.bytes = pl.items.empty() ? 0 : pl.src_off + align_up(pl.src.size() * sizeof(int32_t));
  return pl;
}

dkv_status check_layout(const dkv_params *p, int op, long row_elems, Shape *s) {
  if (!p) return fail(DKV_ERR_INVALID_ARG, "params is NULL");
  if (op < DKV_PACK || op > DKV_FIRST_TOKEN_SCATTER)
    return fail(DKV_ERR_INVALID_ARG, "unknown layout op %d", op);
  if (p->num_seqs < 0) return fail(DKV_ERR_INVALID_ARG, "num_seqs < 0 (%d)", p->num_seqs);
  if (p->ctx_len < 0) return fail(DKV_ERR_INVALID_ARG, "ctx_len < 0 (%d)", p->ctx_len);
  if (!known_dtype(p->dtype))
    return fail(DKV_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  s->dtype = p->dtype;
  if (dkv_status st = check_seqs(p, false, s)) return st;
  const long vec = 16 / (long)elem_size(p->dtype);
  if (row_elems <= 0 || row_elems % vec != 0)
    return fail(DKV_ERR_INVALID_ARG, "row_elems (%ld) must be a positive multiple of %ld", row_elems,
                vec);
  long rows = 0;
  for (int i = 0; i < s->N; ++i) rows += (long)s->sP[i] + s->cu[i + 1] - s->cu[i];
  rows = std::max<long>(rows, (long)s->P + s->T);
  if (rows >= (1L << 31) || row_elems / vec >= (1L << 31) / kRowsPerItem)
    return fail(DKV_ERR_UNSUPPORTED, "layout of %ld rows x %ld elements exceeds the 32-bit row "
                "indices of the kernels", rows, row_elems);
  return DKV_OK;
}

}  // namespace

// ------------------------------------------------------ internal entry points --

namespace dkv {

dkv_status bwd_call(const dkv_params *p, const void *q_resp, const void *k_p, const void *v_p,
                    const void *k_r, const void *v_r, const void *o_r, const float *lse_r,
                    const void *dout_r, void *dq_r, void *dk_r, void *dv_r, float *acc_dk_p,
                    float *acc_dv_p, int acc_flags, void *dk_p, void *dv_p, void *ws,
                    size_t ws_bytes, hipStream_t stream, bool pageable) {
  Shape s;
  dkv_status st = check_params(p, false, &s);
  if (st != DKV_OK) return st;
  if (acc_flags & ~(DKV_ACC_ZERO | DKV_ACC_FINALIZE | DKV_ACC_SPLIT))
    return fail(DKV_ERR_INVALID_ARG, "unknown accumulator flags 0x%x", acc_flags);
  bool need = s.T > 0;
  bool needp = s.P > 0;
  if ((st = check_ptr(q_resp, "q_resp", need)) || (st = check_ptr(k_p, "k_p", need && needp)) ||
      (st = check_ptr(v_p, "v_p", need && needp)) || (st = check_ptr(k_r, "k_r", need)) ||
      (st = check_ptr(v_r, "v_r", need)) || (st = check_ptr(o_r, "o_r", need)) ||
      (st = check_ptr(lse_r, "lse_r", need)) || (st = check_ptr(dout_r, "dout_r", need)) ||
      (st = check_ptr(dq_r, "dq_r", need)) || (st = check_ptr(dk_r, "dk_r", need)) ||
      (st = check_ptr(dv_r, "dv_r", need)) ||
      (st = check_ptr(acc_dk_p, "acc_dk_p", needp)) ||
      (st = check_ptr(acc_dv_p, "acc_dv_p", needp)))
    return st;
  if ((acc_flags & DKV_ACC_FINALIZE) &&
      ((st = check_ptr(dk_p, "dk_p", needp)) || (st = check_ptr(dv_p, "dv_p", needp))))
    return st;
  BwdIO io{};
  io.q = q_resp; io.kc = k_p; io.vc = v_p; io.ko = k_r; io.vo = v_r; io.o = o_r;
  io.dout = dout_r; io.lse = lse_r; io.dq = dq_r; io.dk_own = dk_r; io.dv_own = dv_r;
  io.acc_dk = needp ? acc_dk_p : nullptr; io.acc_dv = needp ? acc_dv_p : nullptr;
  io.acc_rows = s.P; io.flags = acc_flags; io.dk_fin = dk_p; io.dv_fin = dv_p;
  io.with_ctx = true; io.own_to_acc = false;
  return run_bwd(s, io, ws, ws_bytes, stream, pageable ? Staging::kPageable : Staging::kPinned);
}

dkv_status report(dkv_status st, const char *msg) { return fail(st, "%s", msg); }

}  // namespace dkv

// ====================================================================== C ABI ==

extern "C" {

const char *dkv_last_error(void) { return g_err.c_str(); }

const char *dkv_version(void) { return "dkv 0.1 (gfx950)"; }

void dkv_timing_enable(int on) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  t.on = on != 0;
}

void dkv_timing_reset(void) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  for (auto &r : t.recs) {
    hipEventSynchronize(r.b);
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.recs.clear();
}

int dkv_timing_read(const char **names, double *ms, int *launches, int max_entries) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  double sum[kKClasses] = {0};
  int cnt[kKClasses] = {0};
  for (auto &r : t.recs) {
    float x = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&x, r.a, r.b) == hipSuccess) {
      sum[r.cls] += x;
      cnt[r.cls] += 1;
    }
  }
  int n = 0;
  for (int c = 0; c < kKClasses && n < max_entries; ++c) {
    if (!cnt[c]) continue;
    if (names) names[n] = kKernelNames[c];
    if (ms) ms[n] = sum[c];
    if (launches) launches[n] = cnt[c];
    ++n;
  }
  return n;
}

size_t dkv_workspace_size(const dkv_params *p, int which_call) {
  Shape s;
  bool is_ctx = which_call == DKV_CALL_CTX_FWD || which_call == DKV_CALL_CTX_BWD;
  if (which_call < DKV_CALL_CTX_FWD || which_call > DKV_CALL_BWD_SPLIT) {
    fail(DKV_ERR_INVALID_ARG, "unknown call %d", which_call);
    return (size_t)-1;
  }
  if (check_params(p, is_ctx, &s) != DKV_OK) return (size_t)-1;
  if (which_call == DKV_CALL_CTX_FWD || which_call == DKV_CALL_FWD) return plan_fwd(s).bytes;
  const bool with_ctx = which_call == DKV_CALL_BWD || which_call == DKV_CALL_BWD_SPLIT;
  // dkv_ctx_bwd may split its key tiles into row chunks (flags decide): size for them.
  return plan_bwd(s, with_ctx, which_call == DKV_CALL_BWD_SPLIT,
                  which_call == DKV_CALL_CTX_BWD && chunk_own_rows(s)).bytes;
}

dkv_status dkv_ctx_fwd(const dkv_params *p, const void *q, const void *k, const void *v,
                       void *o, float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  dkv_status st = check_params(p, true, &s);
  if (st != DKV_OK) return st;
  bool need = s.T > 0;
  if ((st = check_ptr(q, "q", need)) || (st = check_ptr(k, "k", need)) ||
      (st = check_ptr(v, "v", need)) || (st = check_ptr(o, "o", need)) ||
      (st = check_ptr(lse, "lse", need)))
    return st;
  return run_fwd(s, q, k, v, k, v, o, lse, ws, ws_bytes, stream, Staging::kPinned);
}

dkv_status dkv_fwd(const dkv_params *p, const void *q_resp, const void *k_p, const void *v_p,
                   const void *k_r, const void *v_r, void *o_r, float *lse_r, void *ws,
                   size_t ws_bytes, hipStream_t stream) {
  Shape s;
  dkv_status st = check_params(p, false, &s);
  if (st != DKV_OK) return st;
  bool need = s.T > 0;
  if ((st = check_ptr(q_resp, "q_resp", need)) || (st = check_ptr(k_p, "k_p", need && s.P > 0)) ||
      (st = check_ptr(v_p, "v_p", need && s.P > 0)) || (st = check_ptr(k_r, "k_r", need)) ||
      (st = check_ptr(v_r, "v_r", need)) || (st = check_ptr(o_r, "o_r", need)) ||
      (st = check_ptr(lse_r, "lse_r", need)))
    return st;
  return run_fwd(s, q_resp, k_p, v_p, k_r, v_r, o_r, lse_r, ws, ws_bytes, stream, Staging::kPinned);
}

dkv_status dkv_ctx_bwd(const dkv_params *p, const void *q, const void *k, const void *v,
                       const void *o, const float *lse, const void *dout, void *dq, void *dk,
                       void *dv, float *acc_dk, float *acc_dv, int acc_flags, void *ws,
                       size_t ws_bytes, hipStream_t stream) {
  Shape s;
  dkv_status st = check_params(p, true, &s);
  if (st != DKV_OK) return st;
  if (acc_flags & ~(DKV_ACC_ZERO | DKV_ACC_FINALIZE | DKV_ACC_SPLIT))
    return fail(DKV_ERR_INVALID_ARG,
                "dkv_ctx_bwd accepts DKV_ACC_ZERO | DKV_ACC_FINALIZE | DKV_ACC_SPLIT only");
  if (s.T == 0) return DKV_OK;   // nothing to compute, clear or cast
  const bool use_acc = acc_dk != nullptr || acc_dv != nullptr;
  bool need = true;
  if ((st = check_ptr(q, "q", need)) || (st = check_ptr(k, "k", need)) ||
      (st = check_ptr(v, "v", need)) || (st = check_ptr(o, "o", need)) ||
      (st = check_ptr(lse, "lse", need)) || (st = check_ptr(dout, "dout", need)) ||
      (st = check_ptr(dq, "dq", need)))
    return st;
  if (use_acc) {
    if ((st = check_ptr(acc_dk, "acc_dk", true)) || (st = check_ptr(acc_dv, "acc_dv", true)))
      return st;
    if ((acc_flags & DKV_ACC_FINALIZE) &&
        ((st = check_ptr(dk, "dk", need)) || (st = check_ptr(dv, "dv", need))))
      return st;
  } else {
    if (acc_flags)
      return fail(DKV_ERR_INVALID_ARG, "accumulator flags given without accumulator buffers");
    if ((st = check_ptr(dk, "dk", need)) || (st = check_ptr(dv, "dv", need))) return st;
  }
  BwdIO io{};
  io.q = q; io.kc = k; io.vc = v; io.ko = k; io.vo = v; io.o = o; io.dout = dout; io.lse = lse;
  io.dq = dq; io.dk_own = dk; io.dv_own = dv; io.acc_dk = acc_dk; io.acc_dv = acc_dv;
  io.acc_rows = s.T; io.flags = acc_flags; io.dk_fin = dk; io.dv_fin = dv;
  io.with_ctx = false; io.own_to_acc = use_acc;
  return run_bwd(s, io, ws, ws_bytes, stream, Staging::kPinned);
}

dkv_status dkv_bwd(const dkv_params *p, const void *q_resp, const void *k_p, const void *v_p,
                   const void *k_r, const void *v_r, const void *o_r, const float *lse_r,
                   const void *dout_r, void *dq_r, void *dk_r, void *dv_r, float *acc_dk_p,
                   float *acc_dv_p, int acc_flags, void *dk_p, void *dv_p, void *ws,
                   size_t ws_bytes, hipStream_t stream) {
  return dkv::bwd_call(p, q_resp, k_p, v_p, k_r, v_r, o_r, lse_r, dout_r, dq_r, dk_r, dv_r,
                       acc_dk_p, acc_dv_p, acc_flags, dk_p, dv_p, ws, ws_bytes, stream, false);
}

dkv_status dkv_cast_acc(const dkv_params *p, int32_t rows, const float *acc_dk,
                        const float *acc_dv, void *dk, void *dv, hipStream_t stream) {
  if (!p) return fail(DKV_ERR_INVALID_ARG, "params is NULL");
  if (rows < 0) return fail(DKV_ERR_INVALID_ARG, "rows < 0");
  if (!known_dtype(p->dtype))
    return fail(DKV_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->num_heads_kv <= 0 || p->head_dim <= 0)
    return fail(DKV_ERR_INVALID_ARG, "bad head shape");
  dkv_status st;
  bool need = rows > 0;
  if ((st = check_ptr(acc_dk, "acc_dk", need)) || (st = check_ptr(acc_dv, "acc_dv", need)) ||
      (st = check_ptr(dk, "dk", need)) || (st = check_ptr(dv, "dv", need)))
    return st;
  long n = (long)rows * p->num_heads_kv * p->head_dim;
  hipError_t e;
  e = timed(kKCast, stream, [&] {
    hipError_t r = launch_cast(p->dtype, acc_dk, dk, n, stream);
    return r != hipSuccess ? r : launch_cast(p->dtype, acc_dv, dv, n, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "cast");
  return DKV_OK;
}

size_t dkv_layout_workspace_size(const dkv_params *p, int op) {
  Shape s;
  if (check_layout(p, op, 16 / (p ? (long)elem_size(p->dtype) : 2), &s) != DKV_OK)
    return (size_t)-1;
  return plan_layout(s, op).bytes;
}

dkv_status dkv_layout(const dkv_params *p, int op, int64_t row_elems, const void *in, void *out,
                      void *ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  dkv_status st = check_layout(p, op, (long)row_elems, &s);
  if (st != DKV_OK) return st;
  LayoutPlan pl = plan_layout(s, op);
  if ((st = check_ptr(in, "in", pl.in_rows > 0)) || (st = check_ptr(out, "out", pl.out_rows > 0)))
    return st;
  if ((st = check_ws(ws, ws_bytes, pl.bytes)) != DKV_OK) return st;
  if (pl.items.empty()) return DKV_OK;
  bool capturing = false;
  if ((st = capture_state(stream, Staging::kPinned, &capturing)) != DKV_OK) return st;
  char *wsb = static_cast<char *>(ws);
  {
    StagedImage img(pl.bytes);
    img.put(pl.items_off, pl.items.data(), pl.items.size() * sizeof(RowItem));
    img.put(pl.src_off, pl.src.data(), pl.src.size() * sizeof(int32_t));
    if ((st = upload(img.bytes.data(), img.bytes.size(), wsb, stream)) != DKV_OK) return st;
  }
  const int row_vecs = (int)(row_elems * (long)elem_size(s.dtype) / 16);
  hipError_t e = timed(kKLayout, stream, [&] {
    return launch_row_sum(s.dtype, in, out, reinterpret_cast<const RowItem *>(wsb + pl.items_off),
                          (int)pl.items.size(), reinterpret_cast<const int32_t *>(wsb + pl.src_off),
                          row_vecs, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "layout kernel launch");
  return DKV_OK;
}

}  // extern "C"
