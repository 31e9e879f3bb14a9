/*
 * kda_recoverssm.h -- C ABI of the MI355X (gfx950) KDA RecoverSSM library.
 *
 * The library implements, for Kimi Delta Attention (KDA) layers served with
 * speculative decoding, the two device operations the vLLM Kimi-K3 pages
 * describe:
 *
 *   kda_conv_update_verify  -- the speculative verify of one KDA layer with
 *       the depthwise causal short convolution fused in.  Per request and
 *       head it runs the gated delta rule over the draft positions starting
 *       from the request's checkpoint state, writes the outputs, the per-
 *       position correction and [raw key | raw gate] records, and rolls the
 *       conv state in place.  The checkpoint is only read.
 *       (kernels page `vllm.models.kimi_k3.nvidia.recoverssm.kernels`,
 *       class `CuteRecoverSSMVerify`, method `__call__`; ops page
 *       `vllm/models/kimi_k3/nvidia/ops/recoverssm.py`, functions
 *       `_kda_gate`, `_kda_recurrent_step`, `_kda_recoverssm_verify_kernel`,
 *       `kda_recoverssm_verify`.)
 *
 *   kda_recoverssm_commit   -- folds each request's first n accepted
 *       positions, from those records, into its checkpoint state, for every
 *       layer in one launch; in align mode (prefix caching) it also stores
 *       the state at a completed block boundary.
 *       (kernels page, function `cute_recoverssm_commit`; ops page,
 *       `_commit_kda_state_kernel` and `KDARecoverSSMCommitContext`.)
 *
 *   kda_commit_plan, kda_compact_conv_state -- the two launches that the
 *       ops page's `KDARecoverSSMCommitContext.commit` runs before the
 *       state commit: the per-request plan (commit lengths, final and
 *       boundary slots) and the conv-state compaction.
 *
 *   kda_recoverssm_commit_step -- those three (plan, compaction, commit)
 *       with the same results, in one launch.
 *
 * plus host-only argument checks mirroring the pages' validation
 * (kernels page `_check_layouts`, `can_use_cute_recoverssm`; ops page
 * `kda_recoverssm_verify`, `KDARecoverSSMCommitContext.create/commit`).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are described by kda_tensor: a device pointer, a dtype, and up
 *    to four sizes and strides, strides counted in ELEMENTS.  Every pointer
 *    handed to the library is a device pointer unless stated otherwise.
 *  - The caller owns every buffer.  The library allocates no device memory,
 *    keeps no pointer after a call returns and performs no host/device
 *    synchronisation.  Launches are asynchronous on the given stream (a
 *    hipStream_t passed as void*; NULL = the null stream), so every launch
 *    may be captured in a HIP graph.
 *  - Every entry point returns KDA_OK (0) or a kda_status code; a failing
 *    call launches nothing and leaves a message for kda_last_error() in the
 *    calling thread.  Zero-sized work (batch 0, or no tokens for a verify
 *    without pending_lens) returns KDA_OK without launching.
 *  - Values that live on the device (query lengths, slots, accepted counts,
 *    commit lengths, record rows) are never read by the host.  The kernels
 *    clamp them instead: query length to [0, Q], accepted count to [1, Q],
 *    commit length to [0, Q]; a slot <= null_block_id or >= the pool size is
 *    null; a record row outside [0, rows) writes (verify) or reads (commit)
 *    no records.
 *  - Two requests of one launch must not name the same non-null slot, and a
 *    commit's final slot must not be another request's source slot; the
 *    pages leave these cases undefined and so does this library.
 */
#ifndef KDA_RECOVERSSM_H
#define KDA_RECOVERSSM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 6

/* Status codes. */
typedef enum {
  KDA_OK = 0,
  KDA_E_SHAPE = 1,       /* sizes disagree with each other */
  KDA_E_DTYPE = 2,       /* an element type that is not accepted */
  KDA_E_LAYOUT = 3,      /* strides or alignment of a cache page or
                            parameter tensor (kernels page `_check_layouts`) */
  KDA_E_UNALIGNED = 4,   /* a per-step activation does not start on a
                            16-byte boundary; nothing is launched and the
                            caller may run another implementation (kernels
                            page, `CuteRecoverSSMVerify.__call__` returns
                            False in that case) */
  KDA_E_UNSUPPORTED = 5, /* head dim not in {16,32,64,128}, conv width not
                            4, window Q not in 1..16 */
  KDA_E_CAPACITY = 6,    /* more tokens than batch * Q (ops page,
                            `kda_recoverssm_verify`) */
  KDA_E_DEVICE = 7,      /* a HIP runtime error */
  KDA_E_ARG = 8          /* a required pointer is NULL or a count is
                            negative */
} kda_status;

/* Element types. */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* How the verify hands out its (request, head) work items. */
typedef enum {
  KDA_SCHEDULE_DEFAULT = 0,    /* the library's choice (the fastest measured
                                  for the shape: PER_ITEM up to 65535
                                  requests, else TICKETS) */
  KDA_SCHEDULE_PER_ITEM = 1,   /* one workgroup per item, handed out by the
                                  hardware dispatcher (each XCD takes one
                                  contiguous eighth of the items) */
  KDA_SCHEDULE_TICKETS = 2,    /* persistent workgroups drawing tickets of
                                  items_per_ticket items from work_counter
                                  (the kernels page's design) */
  KDA_SCHEDULE_V_TILES = 3     /* v_tiles workgroups per item, each taking
                                  head_dim / v_tiles rows of the state (the
                                  ops page's verify grid over V blocks,
                                  requests and heads), for batches too small
                                  to fill the GPU; the conv roll of the q
                                  and k channels waits for every V-tile of
                                  the item through an arrival counter in
                                  work_counter.  Head dims 64 and 128,
                                  windows up to 8, no pending_lens.  Same
                                  results, bit for bit, as PER_ITEM. */
} kda_schedule;

/* A strided tensor view.  `stride` is in elements; unused trailing entries
   of shape/stride are ignored. */
typedef struct {
  void* data;
  int32_t dtype;     /* kda_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} kda_tensor;

/* Arguments of kda_conv_update_verify.  H = number of heads, D = head dim
   (= key dim = value dim), T = token rows, Q = spec_query_len (draft window),
   W = 4 conv taps, Lc = Q + W - 2 conv-state length, N state slots, R record
   rows.  "act" is the activation dtype (F32 or BF16) shared by mixed_qkv,
   raw_gate, raw_beta and conv_state. */
typedef struct {
  kda_tensor mixed_qkv;    /* act [T, 3HD]: raw q|k|v projections before the
                              convolution; channel = part*H*D + h*D + d */
  kda_tensor raw_gate;     /* act [T, HD]: gate input before dt_bias */
  kda_tensor raw_beta;     /* act [T, H]: beta before the sigmoid */
  kda_tensor A_log;        /* F32 [H], contiguous */
  kda_tensor dt_bias;      /* F32 [H, D] (or [H*D]), contiguous */
  kda_tensor state;        /* F32 [N, H, D(v), D(k)]: checkpoint pool, read
                              only; strides (any, D*D, D, 1), slot stride a
                              multiple of 16 bytes */
  kda_tensor correction;   /* F32 [R, H, Q, D]: correction record */
  kda_tensor key_gate;     /* F32 or act [R, H, Q, 2D]: [0,D) post-conv raw
                              key, [D,2D) raw gate */
  kda_tensor out;          /* F32 or act [T, HD] */
  kda_tensor conv_state;   /* act; dim-first [N, 3HD, Lc] or token-first
                              [N, Lc, 3HD] (see conv_dim_first); rolled in
                              place */
  kda_tensor conv_weight;  /* F32 or act [3HD, W]; weight[:, W-1] multiplies
                              the newest input */
  const int32_t* query_start_loc;      /* [batch+1] token offsets */
  const int32_t* state_indices;        /* [batch] checkpoint slots */
  const int32_t* num_accepted_tokens;  /* [batch] conv history offset + 1 */
  const int32_t* record_rows;          /* [batch] record row, or NULL: the
                                          request's state slot */
  int32_t* work_counter;   /* device int32[work_counter_len]: [0] is the
                              ticket counter of the ticket schedule,
                              [1 + b * H + h] the arrival counter of request
                              b, head h under the V-tile schedule (fused
                              conv only).  Must be 0 before the first
                              launch; every launch leaves it at 0.  One
                              counter array per launch in flight.  May be
                              NULL for the other schedules. */
  int32_t batch;
  int32_t spec_query_len;  /* Q */
  int32_t null_block_id;   /* slots <= this are null (the ops page imports
                              the value without printing it; the tests
                              use 0) */
  int32_t conv_dim_first;  /* 1: conv_state is [N, 3HD, Lc]; 0: [N, Lc, 3HD] */
  int32_t use_lower_bound; /* 1: g = lower_bound*sigmoid(A x); 0: softplus */
  float lower_bound;
  int32_t max_workgroups;  /* ticket schedule: at most this many
                              workgroups (0 = as many as are resident at
                              once); ignored by the per-item schedule */
  int32_t items_per_ticket; /* ticket schedule: (request, head) items
                               claimed per ticket; 0 = library default */
  int32_t schedule;        /* kda_schedule */
  const int32_t* pending_lens; /* device [batch] or NULL.  When given, the
                              launch first performs the deferred commit of
                              the previous step (state page, deferred
                              commit; ops page `_commit_kda_state_kernel`):
                              the first pending_lens[b] positions (clamped
                              to [0, Q]) recorded in request b's record row
                              are folded into its checkpoint, which is
                              written back in place, and the verify then
                              starts from the updated state and overwrites
                              that row with this step's records.  A request
                              with a live slot and an empty window (no
                              tokens, or T = 0) still folds its pending
                              positions.  Uses the per-item schedule
                              (batch <= 65535). */
  int32_t work_counter_len; /* elements of work_counter; 0 with a counter
                               means 1.  The V-tile schedule of the fused
                               conv verify needs 1 + batch * H. */
  int32_t v_tiles;         /* V-tile schedule: 2, 4 or 8 workgroups per
                              (request, head); 0 = the library's choice */
} kda_verify_args;

/* Arguments of kda_recoverssm_commit.  Per-layer tensors are described by
   device tables of int64 base byte addresses and slot (row) strides in
   elements, as the ops page's commit context builds them; inner strides
   are shared by all layers. */
typedef struct {
  int32_t num_layers;          /* L >= 1 */
  int32_t batch;
  int32_t num_heads;           /* H */
  int32_t head_dim;            /* D */
  int32_t spec_query_len;      /* Q */
  int32_t null_block_id;
  int64_t num_slots;           /* N of every layer's state pool */
  int64_t num_record_rows;     /* R of every layer's records */
  /* device int64[L] tables */
  const int64_t* state_base_addrs;          /* F32 [N, H, D, D] views */
  const int64_t* state_block_strides;
  const int64_t* correction_base_addrs;     /* F32 [R, H, Q, D] views */
  const int64_t* correction_block_strides;
  const int64_t* key_gate_base_addrs;       /* [R, H, Q, 2D] views */
  const int64_t* key_gate_block_strides;
  int64_t state_strides[2];       /* head, row; must be (D*D, D) */
  int64_t correction_strides[2];  /* head, position; dim stride is 1 */
  int64_t key_gate_strides[2];    /* head, position; dim stride is 1 */
  int32_t key_gate_dtype;         /* kda_dtype */
  int32_t max_workgroups;         /* 0: one workgroup per (layer, request,
                                     head); > 0: a persistent grid of at
                                     most this many workgroups */
  const float* A_log;             /* device F32 [L, H] */
  int64_t A_log_strides[2];
  const float* dt_bias;           /* device F32 [L, H, D] */
  int64_t dt_bias_strides[3];
  const int32_t* use_lower_bound; /* device int32 [L]: gate kind per layer */
  const float* lower_bound;       /* device F32 [L] */
  const int32_t* state_indices;   /* device [batch] source slots */
  const int32_t* commit_lens;     /* device [batch] accepted positions */
  const int32_t* final_state_indices; /* device [batch] or NULL: in place */
  const int32_t* record_rows;     /* device [batch] or NULL: source slot */
  /* Optional HOST copy of the six device tables, laid out as int64[6][L] in
     the order above (state bases, state strides, correction bases,
     correction strides, key/gate bases, key/gate strides).  When given,
     the checks verify every layer's alignment; NULL skips those checks. */
  const int64_t* host_tables;
  /* Align mode (ops page `_commit_kda_state_kernel` with ALIGN_MODE): both
     NULL, or both device int32 [batch].  A request that commits and whose
     boundary slot is live also stores, before its final state, the state
     after its first m = boundary_recovery_lens[b] (clamped to [0, n])
     positions at that slot.  Both states come from the source checkpoint
     as it was before the launch; a request's boundary and final slots must
     not be another request's source or destination in the same launch. */
  const int32_t* boundary_state_indices;
  const int32_t* boundary_recovery_lens;
} kda_commit_args;

/* Arguments of kda_commit_plan (ops page: `_prepare_commit_plan_kernel`,
   launched by `KDARecoverSSMCommitContext.commit`; its body is not on the
   pages).  For row b of the batch, with row = request_indices[b] (or b):
     n = num_accepted_tokens[row] clamped to [0, q_b], q_b the window of b
         (0 when state_indices[b] <= null_block_id);
   without a block table: final = state_indices[b], boundary = null id,
   boundary length 0.  With one (prefix caching, one state block per
   mamba_block_size tokens), for c = num_computed_tokens[row] (tokens before
   the window, clamped to >= 0) and n >= 1:
     final = block_table[row][(c + n) / bs], the block that will hold the
             next token (null id when past the table's width);
     when that block starts at P with c < P (the committed tokens completed
     the block before it) and P / bs - 1 is inside the table,
     boundary = block_table[row][P / bs - 1] with boundary length P - c;
     otherwise boundary = null id, length 0.
   A row outside [0, num_request_rows) plans no commit (n = 0). */
typedef struct {
  int32_t batch;
  int32_t spec_query_len;          /* Q */
  int32_t null_block_id;
  int32_t mamba_block_size;        /* align mode: tokens per block, >= Q */
  int32_t num_request_rows;        /* rows of the per-request arrays */
  int32_t block_table_width;       /* align mode: blocks per row */
  int64_t block_table_strides[2];  /* align mode: row, column (elements) */
  const int32_t* num_accepted_tokens;  /* device, per request row */
  const int32_t* request_indices;      /* device [batch] or NULL */
  const int32_t* state_indices;        /* device [batch] */
  const int32_t* query_start_loc;      /* device [batch + 1] */
  const int32_t* block_table;          /* device or NULL (no align) */
  const int32_t* num_computed_tokens;  /* device per request row, or NULL;
                                          given iff block_table is */
  int32_t* commit_lens;                /* device [batch] outputs */
  int32_t* final_state_indices;
  int32_t* boundary_state_indices;
  int32_t* boundary_recovery_lens;
} kda_plan_args;

/* Arguments of kda_compact_conv_state (ops page: `_compact_conv_state_kernel`,
   launched by `KDARecoverSSMCommitContext.commit`; its body is not on the
   pages).  The verify leaves a request's conv state rolled: entry 2 + t
   holds window input t, entries 0 and 1 the two inputs before the window.
   For every layer and every request with a live source slot, n =
   commit_lens[b] (clamped to [0, Q]) >= 1 and a live final slot, entries
   [n - 1, n + 2) of the source (the three inputs before token n of the
   window) are copied to entries [0, 3) of the final slot, so that the next
   verify reads its history with accepted count 1.  In align mode the
   entries [m - 1, m + 2) go to a live boundary slot the same way, when
   m = boundary_recovery_lens[b] (clamped to [0, n]) >= 1.  Other entries
   are not touched; values are copied bit for bit; everything is read
   before anything is written, and the boundary is written first. */
typedef struct {
  int32_t num_layers;
  int32_t batch;
  int32_t spec_query_len;       /* Q: the conv state holds Q + 2 entries */
  int32_t null_block_id;
  int64_t num_slots;            /* N */
  int64_t conv_dim;             /* channels, 3 * H * D */
  int32_t conv_dtype;           /* kda_dtype of every layer's conv state */
  int32_t pad_;
  /* device int64 [4][L]: per layer, the base byte address, then the slot,
     channel and token strides (elements) of its conv state seen dim-first
     as [N, conv_dim, Q + 2] (a token-first state is its transpose). */
  const int64_t* conv_tables;
  const int64_t* host_conv_tables;  /* optional HOST copy, for the checks */
  const int32_t* state_indices;           /* device [batch] */
  const int32_t* commit_lens;             /* device [batch] */
  const int32_t* final_state_indices;     /* device [batch] or NULL */
  const int32_t* boundary_state_indices;  /* both NULL or both given */
  const int32_t* boundary_recovery_lens;
} kda_compact_args;

/* Library ABI version (KDA_ABI_VERSION). */
int kda_abi_version(void);

/* Message of the last failing call in this thread ("" if none). */
const char* kda_last_error(void);

/* Name of a status code. */
const char* kda_status_string(int status);

/* Host-only validation of verify arguments: shapes, dtypes, strides,
   alignment and supported sizes.  Reads no device memory, launches nothing.
   (kernels page `_check_layouts`, `can_use_cute_recoverssm`; ops page
   `kda_recoverssm_verify`.) */
int kda_check_verify(const kda_verify_args* args);

/* Validate, then launch the fused conv update + speculative verify on
   `stream`.  Writes out, correction/key_gate records of the written
   positions, and the rolled conv state; leaves state and every other byte
   unchanged; null requests get +0.0 outputs and nothing else. */
int kda_conv_update_verify(const kda_verify_args* args, void* stream);

/* kda_conv_update_verify for callers that cannot allocate device memory
   (code under HIP graph capture, tight serving loops, harnesses that forbid
   allocation): the same checks, kernels and results, except that the work
   counters (the ticket counter, and the V-tile schedule's arrival counters)
   live in a scratch array of the library instead of args->work_counter,
   which is ignored.  The array holds 1 + 65536 int32 per GPU, is looked up
   (and cleared by a kernel on `stream`) on the first call on each device,
   and is kept until the process ends.  Every launch leaves it at zero, but
   it is shared: calls that overlap on one GPU (two streams, or two threads)
   race on it.  A V-tile launch of more than 65536 (request, head) items is
   refused with KDA_E_CAPACITY before any device call.  Allocates nothing. */
int kda_conv_update_verify_noalloc(const kda_verify_args* args, void* stream);

/* The unfused verify (ops page, `kda_recoverssm_verify` and
   `_kda_recoverssm_verify_kernel`): the same as kda_conv_update_verify
   except that mixed_qkv [T, 3HD] already holds the convolved q | k | v
   (the three column blocks, channel = part*H*D + h*D + d) and the key
   record stores that k as given.  conv_state, conv_weight and
   num_accepted_tokens are not used (they may be empty / NULL). */
int kda_check_verify_qkv(const kda_verify_args* args);
int kda_recoverssm_verify_qkv(const kda_verify_args* args, void* stream);

/* Host-only validation of commit arguments (ops page
   `KDARecoverSSMCommitContext.create` and `.commit`). */
int kda_check_commit(const kda_commit_args* args);

/* Validate, then launch the multi-layer commit on `stream`: for every layer
   and request with a non-null source slot, a non-null final slot, a valid
   record row and n = commit length > 0, the checkpoint of every head
   becomes S_n = S_0 * prod_t diag(exp g_t) + sum_t c_t k_hat_t^T
   * prod_{s>t} diag(exp g_s) over t < n, stored at the final slot. */
int kda_recoverssm_commit(const kda_commit_args* args, void* stream);

/* Host-only validation of the plan arguments, then its launch on `stream`
   (one thread per request; writes only the four output arrays). */
int kda_check_commit_plan(const kda_plan_args* args);
int kda_commit_plan(const kda_plan_args* args, void* stream);

/* Host-only validation of the compaction arguments, then its launch on
   `stream` (one thread per layer, request and channel). */
int kda_check_compact_conv(const kda_compact_args* args);
int kda_compact_conv_state(const kda_compact_args* args, void* stream);

/* The whole of the ops page's `KDARecoverSSMCommitContext.commit` in one
   launch: the results of kda_commit_plan(plan), then, when `compact` is not
   NULL, kda_compact_conv_state(compact), then kda_recoverssm_commit(commit),
   bit for bit.  Every (layer, request, head) workgroup of the commit plans
   its request itself (the layer-0, head-0 one writes the plan's four
   outputs) and copies that head's conv histories (its q, k and v channels)
   before its state fold.
   The three blocks must describe the calls the separate path would make:
   one batch, window and null id; the commit's state_indices, commit_lens
   and final_state_indices (and, iff the plan has a block table, its
   boundary pair) are the plan's state_indices and output pointers, and so
   are the compaction's; the compaction covers the commit's layers and slot
   count with conv_dim = 3 * num_heads * head_dim.  Otherwise KDA_E_ARG.
   The plan's output arrays are written, never read, by the launch.  The
   slot rules of the separate calls hold: no request's final or boundary
   slot is another request's source or destination. */
int kda_check_commit_step(const kda_commit_args* commit,
                          const kda_plan_args* plan,
                          const kda_compact_args* compact);
int kda_recoverssm_commit_step(const kda_commit_args* commit,
                               const kda_plan_args* plan,
                               const kda_compact_args* compact,
                               void* stream);

/* Launch a one-workgroup kernel that sets counter[0..n) to 0 on `stream`
   (for a counter left non-zero by an aborted launch).  Uses no memset
   node, so it may be captured in a graph. */
int kda_reset_counter(int32_t* counter, int32_t n, void* stream);

/* Kernel timing without a profiler, for callers that measure each kernel's
   own duration (an event recorded on the stream around a launch also counts
   the gap the event's own marker adds before the next dispatch).  Arms the
   calling thread: the next `launches` verify, commit, plan or compaction
   kernels that library calls on this thread launch are dispatched with
   hipExtLaunchKernel, `start_event` (a hipEvent_t, may be NULL) recording
   the start of the first of them and `stop_event` (may be NULL) the end of
   the last.  The counter-clearing kernels (kda_reset_counter, the first
   use of the no-allocation entry point's array on a device) are not
   counted.  launches = 0 disarms.  If `pending` is not NULL it receives
   the number of launches the previous arming was still waiting for (0 when
   every armed launch happened, so its stop event was recorded).  The
   events stay the caller's; do not arm the thread while it captures a
   graph.  KDA_E_ARG if launches < 0 (the previous arming is then kept). */
int kda_set_launch_events(void* start_event, void* stop_event,
                          int32_t launches, int32_t* pending);

#ifdef __cplusplus
}
#endif
#endif /* KDA_RECOVERSSM_H */
