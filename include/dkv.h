/*
 * dkv.h -- C ABI of libdkv: DualKV shared-prompt attention on AMD MI355X (gfx950).
 *
 * The method ("DualKV: Shared-Prompt Flash Attention for Efficient RL Training with
 * Large Rollouts and Long Contexts", arXiv 2605.15422) computes exact causal
 * attention for N responses that share one P-token prompt.  The batch is packed
 * with a single prompt copy (§2.2, eq. (5)): prompt rows, then response 1..N.  The
 * work splits into two calls (§2.2 "two-call decomposition"):
 *
 *   Call 1  dkv_ctx_fwd / dkv_ctx_bwd  causal self-attention over the single prompt
 *                                     copy (eq. (3)).  With several sequences it is
 *                                     plain varlen causal attention, which is also
 *                                     how the N-copy packing of §2.1 (eq. (2)) runs.
 *   Call 2  dkv_fwd / dkv_bwd          every response attends to the shared K_P,V_P
 *                                     and to its own K_Ri,V_Ri under the causal mask
 *                                     shifted by P (eq. (4), §3.1).
 *
 * The gradient of the shared prompt K_P,V_P is the Call-1 term plus the sum of the
 * N Call-2 terms (eq. (6)); both calls add into one caller-owned fp32 accumulator,
 * which is cast to the tensor dtype exactly once (§3.2 "fp32 atomic accumulation").
 *
 * Conventions (all entry points)
 *   - Tensors are caller-owned, contiguous, token-major device buffers:
 *       queries / outputs / output grads  [tokens, Hq,  d]
 *       keys / values / their grads       [tokens, Hkv, d]
 *       LSE                               [Hq, tokens] fp32, natural log
 *     in the dtype named by dkv_params.dtype (bf16, fp16 or fp32).  Device pointers must
 *     be 16-byte aligned.
 *   - The library never allocates or frees device memory.  Scratch space comes from
 *     `ws` (device memory, `ws_bytes` long, 256-byte aligned), sized by
 *     dkv_workspace_size() for the same parameters and call.
 *   - Calls only enqueue work on `stream` and return; they never wait for the device.
 *     Work lists are copied from pinned host buffers that are reused once their copy
 *     has completed (polled); when all are in flight another is allocated, so the
 *     pinned pool grows with the caller's run-ahead instead of blocking.  The returned
 *     status reports argument validation and launch errors; a fault inside a kernel
 *     surfaces at the caller's next synchronization.
 *   - A non-OK status leaves a message retrievable with dkv_last_error() (per host
 *     thread).  Validation happens before any device work is enqueued, so an
 *     invalid call enqueues nothing.
 *   - Concurrent calls on different streams must not share a workspace.
 *   - Calls may be captured into a HIP graph (hipStreamBeginCapture on `stream`, any
 *     capture mode).  The work-list copy and the kernels become nodes of the graph, and
 *     every replay computes the call again on the buffers and shapes it was captured
 *     with: the buffers' contents may change between replays, the shapes (and the host
 *     cu_seqlens) may not.  The pinned buffer that a captured call copies its lists
 *     from is reserved for that graph until the process ends (32 bytes per work item
 *     plus the sequence and head tables: under 1 MB for the Qwen3-8B-shaped
 *     micro-batch).  The workspace of a captured call belongs to the graph: calls that
 *     may run at the same time as a replay need another.  Per-kernel timing records
 *     nothing under capture.  dkv_bwd_noalloc refuses a capturing stream.
 */
#ifndef DKV_H
#define DKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DKV_OK = 0,
    DKV_ERR_INVALID_ARG = 1,   /* inconsistent shapes, bad cu_seqlens, null pointers */
    /* valid but not implemented: head_dim 192, 256 or 512 in fp32, Hq / Hkv above 128
       (32 at head_dim 192, 256, 512), or (bf16 / fp16) a sequence whose query rows, plus
       64, exceed 2^31 bytes or Hq * tokens above 2^29 -- the kernels' 32-bit row
       offsets */
    DKV_ERR_UNSUPPORTED = 2,
    DKV_ERR_WORKSPACE = 3,     /* ws too small or misaligned */
    DKV_ERR_HIP = 4            /* a HIP runtime call failed */
} dkv_status;

/* Tensor element types.  bf16 and fp16 run the same 16-bit MFMA kernels (fp32
   accumulation, softmax and LSE in fp32); fp16 is the precision of the paper's kernel
   benchmark (§4.1, Table 1). */
typedef enum { DKV_BF16 = 0, DKV_FP32 = 1, DKV_FP16 = 2 } dkv_dtype;

/* Which call a workspace is sized for. */
typedef enum {
    DKV_CALL_CTX_FWD = 0,
    DKV_CALL_FWD = 1,
    DKV_CALL_CTX_BWD = 2,
    DKV_CALL_BWD = 3,
    DKV_CALL_BWD_SPLIT = 4     /* dkv_bwd with DKV_ACC_SPLIT (adds the slices) */
} dkv_call;

/* Flags of the shared-prompt gradient accumulator (dkv_ctx_bwd / dkv_bwd). */
enum {
    DKV_ACC_ZERO = 1,      /* clear acc_dk_p / acc_dv_p before adding this call's terms */
    DKV_ACC_FINALIZE = 2,  /* after adding, cast the accumulator into dk_p / dv_p once */
    /* dkv_bwd.  §3.2 Stage 1 resolves the N-way write to the shared dK_c / dV_c
       with fp32 atomic adds into a scratch buffer (the default here too).  This flag
       resolves it without atomics, still summing in fp32 and casting once:
       the responses are taken in S chunks of ceil(N / S) sequences
       (S = min(N, 8)); a chunk's partial dK_P / dV_P, summed in registers, is stored
       into its own fp32 slice of the workspace (size it with DKV_CALL_BWD_SPLIT), and
       one kernel then adds the slices to the accumulator in slice order.  No atomics
       touch the accumulator, so for given inputs and call order dk_p / dv_p are
       bitwise reproducible when dkv_ctx_bwd gets the flag too.  Workspace:
       2 * S * P * Hkv * d * 4 bytes more.
       dkv_ctx_bwd (with an accumulator): without this flag, when the call's key tiles
       are few (fewer than 1024 tiles times kv heads), the query rows of a long tile may
       be split over several work items that each add their partial sums into the
       accumulator (fp32 atomics), which fills the GPU; with it every element of the
       Call-1 term has one writer. */
    DKV_ACC_SPLIT = 4
};

typedef struct {
    /* Number of sequences.  dkv_fwd/dkv_bwd: N responses.  dkv_ctx_*: number of
       independent causal sequences (1 for Call 1 over the prompt; N for the N-copy
       packing of eq. (2)). */
    int32_t num_seqs;
    /* P, the shared prompt length (context_seqlen of §3).  dkv_fwd/dkv_bwd only:
       response row r sits at logical position P + r.  Must be 0 for dkv_ctx_*. */
    int32_t ctx_len;
    int32_t num_heads_q;       /* Hq, a multiple of Hkv (grouped-query attention) */
    int32_t num_heads_kv;      /* Hkv; q-head h reads kv head h / (Hq / Hkv) unless
                                  kv_head_of_q says otherwise */
    /* d: 64, 96, 128, 192, 256 or 512 (the head dims of the paper's kernel checks,
       App. E.1, and the d = 512 / d = 256 global / sliding-window layers of §3); fp32
       tensors take 64, 96 and 128 */
    int32_t head_dim;
    /* -1: global causal.  w >= 0: key at logical position j is visible from the query
       at logical position t iff t - w <= j <= t (applies to the prompt region too). */
    int32_t window_left;
    float softmax_scale;       /* <= 0 selects 1/sqrt(head_dim) (eqs. (2)-(4)) */
    int32_t dtype;             /* dkv_dtype of every tensor except LSE/accumulators */
    /* Prefix sums of the per-sequence query lengths, int32 [num_seqs + 1] with
       cu[0] = 0, non-decreasing (zero-length sequences allowed).  The host copy is
       read during the call: it is validated, drives the tile schedule, and is staged
       into the workspace with the work lists, which is where the kernels read the
       sequence bounds.  cu_seqlens_dev is optional (may be NULL) and not read: a device
       copy that disagreed with the host copy could otherwise send the kernels outside
       the tensors the host copy describes. */
    const int32_t *cu_seqlens_host;
    const int32_t *cu_seqlens_dev;
    /* Prompt groups (dkv_fwd / dkv_bwd only; must be 0 for dkv_ctx_*).  A micro-batch
       may hold the responses of several prompts, each group with its own shared
       context K/V and its own sequences (§2.2 "Data pipeline": groups are processed
       independently, each with its own context KV and cu_seqlens).
         0: one group -- every sequence shares the ctx_len prompt rows.
         G >= 1: group j's prompt is rows ctx_cu_host[j] .. ctx_cu_host[j+1]-1 of
           k_p / v_p (and of acc_dk_p / acc_dv_p, dk_p / dv_p), and it is shared by
           sequences group_seq_cu_host[j] .. group_seq_cu_host[j+1]-1 of cu_seqlens.
           Both arrays are host int32 [G + 1], start at 0 and do not decrease;
           ctx_cu_host[G] == ctx_len and group_seq_cu_host[G] == num_seqs.  Empty
           prompts and groups without sequences are allowed.  A response row r of a
           sequence of group j sits at logical position (ctx_cu_host[j+1] -
           ctx_cu_host[j]) + r and sees only its own group's prompt.  The Call-1 term
           of every group is the plain varlen dkv_ctx_* call with cu_seqlens =
           ctx_cu_host. */
    int32_t num_groups;
    const int32_t *ctx_cu_host;
    const int32_t *group_seq_cu_host;
    /* Grouped-query attention head map (§3.1 and §4.1: several query heads share one
       key/value head; the paper's Qwen3-8B dimensions use 4 query heads per kv head).
       NULL: q-head h reads kv head h / (Hq / Hkv).  Otherwise a host int32 [Hq] array
       read during the call: q-head h reads kv head kv_head_of_q[h], in [0, Hkv), and
       every kv head must be named by exactly Hq / Hkv q-heads (DKV_ERR_INVALID_ARG
       otherwise).  It applies to every tensor of the call: O, LSE and the gradients
       stay indexed by q-head and kv head as given. */
    const int32_t *kv_head_of_q;
} dkv_params;

/* Bytes of device workspace the given call needs for these parameters (0 means
   none; a valid pointer is still fine).  Returns (size_t)-1 for invalid params.  The
   workspace holds the call's work lists and tables (staged from pinned host memory on
   the call's stream) and, for the backward calls, the per-row terms -D and -LSE / scale
   ([Hq, tokens] fp32 each) and, with DKV_ACC_SPLIT, the accumulator slices. */
size_t dkv_workspace_size(const dkv_params *p, int which_call);

/*
 * Call 1 forward, eq. (3) -- causal self-attention of each sequence of
 * cu_seqlens (varlen).  q [T, Hq, d], k/v [T, Hkv, d], T = cu[num_seqs];
 * writes o [T, Hq, d] and lse [Hq, T].
 */
dkv_status dkv_ctx_fwd(const dkv_params *p, const void *q, const void *k, const void *v,
                       void *o, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Call 2 forward, eq. (4) and §3.1 -- response rows of sequence i attend to the
 * shared prompt keys [0, P) and to their own preceding response keys, as one
 * online softmax over both regions.  q_resp [T_R, Hq, d]; k_p/v_p [P, Hkv, d];
 * k_r/v_r [T_R, Hkv, d]; T_R = cu[num_seqs].  Writes o_r [T_R, Hq, d] and
 * lse_r [Hq, T_R].
 */
dkv_status dkv_fwd(const dkv_params *p, const void *q_resp, const void *k_p,
                   const void *v_p, const void *k_r, const void *v_r, void *o_r,
                   float *lse_r, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Call 1 backward -- gradients of eq. (3) for upstream gradient dout (for the
 * single prompt copy: the sum of the N copies' prompt-row gradients, Appendix A.5).
 * Inputs as in dkv_ctx_fwd plus o, lse (from the forward) and dout [T, Hq, d].
 * Writes dq [T, Hq, d].  Key/value gradients:
 *   - acc_dk / acc_dv non-NULL (fp32 [T, Hkv, d]): added into the accumulator
 *     (cleared first with DKV_ACC_ZERO; cast into dk/dv with DKV_ACC_FINALIZE;
 *     DKV_ACC_SPLIT keeps one writer per element, see the flags above).  With one
 *     sequence over the prompt this is the Call-1 term of eq. (6).
 *   - acc_dk / acc_dv NULL: written directly to dk / dv [T, Hkv, d] (plain varlen
 *     causal backward, e.g. the N-copy packing).
 */
dkv_status dkv_ctx_bwd(const dkv_params *p, const void *q, const void *k, const void *v,
                       const void *o, const float *lse, const void *dout, void *dq,
                       void *dk, void *dv, float *acc_dk, float *acc_dv, int acc_flags,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Call 2 backward, §3.2 -- gradients of eq. (4).  Inputs as in dkv_fwd plus o_r,
 * lse_r and dout_r [T_R, Hq, d].  Writes dq_r [T_R, Hq, d] and dk_r/dv_r
 * [T_R, Hkv, d] directly; adds the N responses' prompt-key terms into
 * acc_dk_p / acc_dv_p (fp32 [P, Hkv, d], required when P > 0).  With
 * DKV_ACC_FINALIZE, casts the accumulator into dk_p / dv_p [P, Hkv, d] once all
 * terms are in.
 */
dkv_status dkv_bwd(const dkv_params *p, const void *q_resp, const void *k_p,
                   const void *v_p, const void *k_r, const void *v_r, const void *o_r,
                   const float *lse_r, const void *dout_r, void *dq_r, void *dk_r,
                   void *dv_r, float *acc_dk_p, float *acc_dv_p, int acc_flags,
                   void *dk_p, void *dv_p, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * dkv_bwd without a workspace, for callers that cannot allocate (code that must not
 * call hipMalloc, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, validation, results and accumulator protocol as dkv_bwd; the scratch space
 * dkv_bwd takes from `ws` comes instead from a device array inside the library of
 * 64 MiB per GPU (held from the first such call on a device until the process ends),
 * and the work lists are copied from pageable host memory, a copy HIP performs
 * synchronously: the call returns once the lists have left the host, and it allocates
 * neither device nor pinned host memory.  A call whose dkv_workspace_size (DKV_CALL_BWD,
 * or DKV_CALL_BWD_SPLIT with DKV_ACC_SPLIT) exceeds 64 MiB returns DKV_ERR_UNSUPPORTED
 * and enqueues nothing (the Qwen3-8B-shaped micro-batch, 131 072 response rows x 32
 * q-heads, needs about 36 MiB).  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other host threads) race, so run them one
 * after another.  A pageable copy cannot be captured into a graph: on a capturing
 * stream the call returns DKV_ERR_UNSUPPORTED and enqueues nothing.
 */
dkv_status dkv_bwd_noalloc(const dkv_params *p, const void *q_resp, const void *k_p,
                           const void *v_p, const void *k_r, const void *v_r, const void *o_r,
                           const float *lse_r, const void *dout_r, void *dq_r, void *dk_r,
                           void *dv_r, float *acc_dk_p, float *acc_dv_p, int acc_flags,
                           void *dk_p, void *dv_p, hipStream_t stream);

/*
 * The single cast of §3.2 (Stage 2) on its own: acc_dk/acc_dv fp32 [rows, Hkv, d]
 * -> dk/dv [rows, Hkv, d] in p->dtype, round-to-nearest-even (a copy for fp32).
 */
dkv_status dkv_cast_acc(const dkv_params *p, int32_t rows, const float *acc_dk,
                        const float *acc_dv, void *dk, void *dv, hipStream_t stream);

/*
 * Layout conversions of per-token rows between the two packings of a micro-batch
 * (any per-token tensor: hidden states, Q/K/V, their gradients), so that every
 * per-token operation of the model can run on the single-prompt packing (§2.2,
 * App. A.3: all per-token operations process P + sum_i R_i tokens):
 *   N-copy packing (§2.1, eq. (1)): for each sequence i in order, its prompt's rows
 *     then its own R_i rows -- sum_i (P_g(i) + R_i) rows.
 *   single-prompt packing (eq. (5)): every prompt once (group order, as ctx_cu_host
 *     lays them out; one prompt of ctx_len rows without groups), then every response
 *     (cu_seqlens order) -- ctx_len + T_R rows.
 * Rows are row_elems elements of p->dtype (a multiple of 16 bytes); in/out are
 * 16-byte aligned device buffers that must not overlap.  The head fields of p are
 * not used.  Ops:
 *   DKV_PACK        N-copy -> single-prompt.  A prompt row comes from its group's first
 *                   copy (every copy holds the same prompt rows, App. A.2); a prompt
 *                   whose group has no response is not in the N-copy packing and is
 *                   written as zeros.
 *   DKV_UNPACK      single-prompt -> N-copy: every copy receives its group's prompt.
 *   DKV_UNPACK_BWD  the adjoint of DKV_UNPACK, for gradients: a prompt row receives
 *                   the sum over its group's copies (App. A.5: the shared prompt
 *                   collects every branch's gradient), accumulated in fp32 in sequence
 *                   order and rounded once; response rows are copied.
 *   DKV_FIRST_TOKEN_GATHER  out [T_R, row]: the hidden state that predicts each
 *                   response token -- for token r > 0 of response i its row r - 1, for
 *                   r = 0 the last row of its group's prompt (§2.3: the last prompt
 *                   token predicts the first token of every response of its group);
 *                   zeros for a first token whose prompt is empty.
 *   DKV_FIRST_TOKEN_SCATTER  the adjoint of the gather, in [T_R, row] -> out
 *                   [ctx_len + T_R, row]: the last row of each prompt receives the sum
 *                   (fp32, sequence order, one rounding) of its responses' first-token
 *                   gradients, a response row r the gradient of token r + 1, and every
 *                   other row zero.
 * Workspace (work lists) from dkv_layout_workspace_size(p, op).  Rows above 2^31 or
 * rows of 2^31 / 16 vectors or more return DKV_ERR_UNSUPPORTED.
 */
typedef enum {
    DKV_PACK = 0,
    DKV_UNPACK = 1,
    DKV_UNPACK_BWD = 2,
    DKV_FIRST_TOKEN_GATHER = 3,
    DKV_FIRST_TOKEN_SCATTER = 4
} dkv_layout_op;
size_t dkv_layout_workspace_size(const dkv_params *p, int op);
dkv_status dkv_layout(const dkv_params *p, int op, int64_t row_elems, const void *in, void *out,
                      void *ws, size_t ws_bytes, hipStream_t stream);
/*
 * Per-kernel timing, a profiling aid.  While enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on its own stream.
 * dkv_timing_read() waits for those events and reports, per kernel class, the
 * summed milliseconds and the launch count since the last reset; it returns the
 * number of classes written (at most max_entries).  Names are static strings.
 * Not thread-safe against concurrent launches from other host threads.
 */
void dkv_timing_enable(int on);
void dkv_timing_reset(void);
int dkv_timing_read(const char **names, double *ms, int *launches, int max_entries);

/* Message for the last non-OK status on this host thread ("" if none). */
const char *dkv_last_error(void);

/* Library version string. */
const char *dkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DKV_H */
