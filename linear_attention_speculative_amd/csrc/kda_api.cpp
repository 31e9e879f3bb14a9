// Host side of the KDA RecoverSSM library: argument checks (mirroring the
// validation of the kernels page's `_check_layouts` and
// `can_use_cute_recoverssm` and the ops page's `kda_recoverssm_verify` and
// `KDARecoverSSMCommitContext.create/commit`), translation of the public
// descriptors into launch parameters, and the exported C entry points.
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>

#include <string>

#include "kda_internal.hpp"
#include "kda_recoverssm.h"

namespace kda {

LaunchTiming& launch_timing() {
  thread_local LaunchTiming t;
  return t;
}

}  // namespace kda

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int elem_size(int32_t dt) {
  return dt == KDA_F32 ? 4 : (dt == KDA_BF16 ? 2 : 0);
}

bool aligned(const void* p, uintptr_t a) {
  return reinterpret_cast<uintptr_t>(p) % a == 0;
}

const char* dt_name(int32_t dt) {
  return dt == KDA_F32 ? "float32" : (dt == KDA_BF16 ? "bfloat16" : "?");
}

bool supported_head_dim(int64_t d) {
  return d == 16 || d == 32 || d == 64 || d == 128;
}

// Checks ndim, non-negative sizes, known dtype and a data pointer.
int check_desc(const kda_tensor& t, const char* name, int ndim) {
  if (t.ndim != ndim)
    return fail(KDA_E_SHAPE, "%s must have %d dimensions (got %d)", name,
                ndim, t.ndim);
  for (int i = 0; i < ndim; ++i)
    if (t.shape[i] < 0)
      return fail(KDA_E_SHAPE, "%s has a negative size", name);
  if (elem_size(t.dtype) == 0)
    return fail(KDA_E_DTYPE, "%s has an unknown dtype code %d", name,
                t.dtype);
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) numel *= t.shape[i];
  if (t.data == nullptr && numel > 0)
    return fail(KDA_E_ARG, "%s has no data pointer", name);
  return KDA_OK;
}

bool shape_is(const kda_tensor& t, int64_t a, int64_t b, int64_t c = -1,
              int64_t d = -1) {
  if (t.shape[0] != a || t.shape[1] != b) return false;
  if (c >= 0 && t.shape[2] != c) return false;
  if (d >= 0 && t.shape[3] != d) return false;
  return true;
}

struct VerifyPlan {
  kda::VerifyParams p;
  int D = 0;
  bool act_bf16 = false;
  bool noop = false;
  int grid = 0;
  int schedule = 0;
};

// V-tiles per (request, head) item for the V-tile schedule when the caller
// leaves the count to the library: enough workgroups to cover the compute
// units when the items alone would not.
int default_vtiles(int64_t items) {
  return items <= 64 ? 8 : items <= 128 ? 4 : 2;
}

#define KDA_TRY(expr)             \
  do {                            \
    int rc_ = (expr);             \
    if (rc_ != KDA_OK) return rc_; \
  } while (0)

// conv: the fused conv update (kda_conv_update_verify); otherwise mixed_qkv
// already holds the convolved q | k | v (kda_recoverssm_verify_qkv) and the
// conv state, taps and accepted counts are not used.  scratch_len > 0: the
// library supplies the work counters (that many), a->work_counter is
// ignored and plan->p.counter is left for the caller to set.
int plan_verify(const kda_verify_args* a, VerifyPlan* plan, bool conv,
                int64_t scratch_len = 0) {
  if (a == nullptr) return fail(KDA_E_ARG, "verify arguments are NULL");
  if (a->batch < 0) return fail(KDA_E_ARG, "batch is negative");
  const int64_t Q = a->spec_query_len;
  if (Q < 1 || Q > kda::kMaxWindow)
    return fail(KDA_E_UNSUPPORTED,
                "KDA RecoverSSM verify supports 1 to %d draft positions per "
                "step (got %lld)",
                kda::kMaxWindow, (long long)Q);

  // Parameters and pool: heads, head dim, slots.
  KDA_TRY(check_desc(a->A_log, "A_log", 1));
  KDA_TRY(check_desc(a->state, "state", 4));
  const kda_tensor& S = a->state;
  const int64_t H = a->A_log.shape[0];
  const int64_t N = S.shape[0];
  const int64_t D = S.shape[3];
  if (H < 1) return fail(KDA_E_SHAPE, "A_log must hold one value per head");
  if (S.dtype != KDA_F32)
    return fail(KDA_E_DTYPE, "the checkpoint state must be float32");
  if (!supported_head_dim(D))
    return fail(KDA_E_UNSUPPORTED,
                "head dim %lld is not supported (16, 32, 64 or 128)",
                (long long)D);
  if (S.shape[1] != H || S.shape[2] != D)
    return fail(KDA_E_SHAPE,
                "checkpoint shape [%lld, %lld, %lld, %lld] does not match "
                "[slots, heads=%lld, %lld, %lld]",
                (long long)S.shape[0], (long long)S.shape[1],
                (long long)S.shape[2], (long long)S.shape[3], (long long)H,
                (long long)D, (long long)D);
  if (N < 1) return fail(KDA_E_SHAPE, "the state pool has no slots");
  if (S.stride[1] != D * D || S.stride[2] != D || S.stride[3] != 1 ||
      (S.stride[0] * 4) % 16 != 0)
    return fail(KDA_E_LAYOUT,
                "state strides (%lld, %lld, %lld, %lld) need contiguous "
                "heads and 16-byte aligned slots",
                (long long)S.stride[0], (long long)S.stride[1],
                (long long)S.stride[2], (long long)S.stride[3]);
  if (a->A_log.dtype != KDA_F32 || a->A_log.stride[0] != 1)
    return fail(a->A_log.dtype != KDA_F32 ? KDA_E_DTYPE : KDA_E_LAYOUT,
                "A_log must be a contiguous float32 vector");
  const kda_tensor& dtb = a->dt_bias;
  if (dtb.ndim != 1 && dtb.ndim != 2)
    return fail(KDA_E_SHAPE, "dt_bias must be [H*D] or [H, D]");
  KDA_TRY(check_desc(dtb, "dt_bias", dtb.ndim));
  if (dtb.dtype != KDA_F32)
    return fail(KDA_E_DTYPE, "dt_bias must be float32");
  if (dtb.ndim == 1 ? (dtb.shape[0] != H * D || dtb.stride[0] != 1)
                    : (dtb.shape[0] != H || dtb.shape[1] != D ||
                       dtb.stride[1] != 1 || dtb.stride[0] != D))
    return fail(KDA_E_SHAPE,
                "dt_bias must hold heads*head_dim contiguous values");

  // Activations.
  KDA_TRY(check_desc(a->mixed_qkv, "mixed_qkv", 2));
  KDA_TRY(check_desc(a->raw_gate, "raw_gate", 2));
  KDA_TRY(check_desc(a->raw_beta, "raw_beta", 2));
  KDA_TRY(check_desc(a->out, "out", 2));
  const int32_t act = a->mixed_qkv.dtype;
  const int64_t T = a->mixed_qkv.shape[0];
  const int64_t HD = H * D;
  if (a->raw_gate.dtype != act || a->raw_beta.dtype != act)
    return fail(KDA_E_DTYPE,
                "mixed_qkv, raw_gate and raw_beta must share one dtype");
  if (!shape_is(a->mixed_qkv, T, 3 * HD))
    return fail(KDA_E_SHAPE, "mixed_qkv must be [T, 3*H*D] = [%lld, %lld]",
                (long long)T, (long long)(3 * HD));
  if (!shape_is(a->raw_gate, T, HD) || !shape_is(a->raw_beta, T, H))
    return fail(KDA_E_SHAPE,
                "KDA RecoverSSM gate or beta shape is incompatible");
  if (!shape_is(a->out, T, HD))
    return fail(KDA_E_SHAPE, "KDA RecoverSSM output shape is incompatible");
  if (a->out.dtype != KDA_F32 && a->out.dtype != act)
    return fail(KDA_E_DTYPE, "out must be float32 or the activation dtype");
  if (a->mixed_qkv.stride[1] != 1 || a->raw_gate.stride[1] != 1 ||
      a->raw_beta.stride[1] != 1 || a->out.stride[1] != 1)
    return fail(KDA_E_LAYOUT,
                "KDA RecoverSSM activation and output heads must be "
                "contiguous");

  // Records.
  KDA_TRY(check_desc(a->correction, "correction", 4));
  KDA_TRY(check_desc(a->key_gate, "key_gate", 4));
  const int64_t R = a->correction.shape[0];
  if (!shape_is(a->correction, R, H, Q, D))
    return fail(KDA_E_SHAPE,
                "KDA RecoverSSM correction buffer needs shape [rows, %lld, "
                "%lld, %lld]",
                (long long)H, (long long)Q, (long long)D);
  if (!shape_is(a->key_gate, R, H, Q, 2 * D))
    return fail(KDA_E_SHAPE,
                "KDA RecoverSSM key/gate buffer needs shape [%lld, %lld, "
                "%lld, %lld]",
                (long long)R, (long long)H, (long long)Q, (long long)(2 * D));
  if (a->correction.dtype != KDA_F32)
    return fail(KDA_E_DTYPE,
                "KDA RecoverSSM correction buffer must use float32");
  if (a->key_gate.dtype != KDA_F32 && a->key_gate.dtype != act)
    return fail(KDA_E_DTYPE,
                "the key/gate buffer must be float32 or the activation "
                "dtype");
  if (a->correction.stride[3] != 1 || a->key_gate.stride[3] != 1)
    return fail(KDA_E_LAYOUT, "record rows must be contiguous");

  // Conv state and weight.
  const kda_tensor no_tensor{};
  const kda_tensor& cs = conv ? a->conv_state : no_tensor;
  const kda_tensor& cw = conv ? a->conv_weight : no_tensor;
  const int64_t C3 = 3 * HD;
  const int64_t Lc = !conv ? 0 : a->conv_dim_first ? cs.shape[2] : cs.shape[1];
  if (conv) {
    KDA_TRY(check_desc(a->conv_state, "conv_state", 3));
    KDA_TRY(check_desc(a->conv_weight, "conv_weight", 2));
    const int64_t cdim = a->conv_dim_first ? cs.shape[1] : cs.shape[2];
    if (cs.shape[0] != N || cdim != C3)
      return fail(KDA_E_SHAPE,
                  "conv state must be [slots=%lld, %lld, Lc] (dim first) or "
                  "[slots, Lc, %lld] (token first)",
                  (long long)N, (long long)C3, (long long)C3);
    if (cs.dtype != act)
      return fail(KDA_E_DTYPE,
                  "the conv state must use the activation dtype (%s)",
                  dt_name(act));
    if (Lc - Q + 2 != kda::kConvWidth)
      return fail(KDA_E_UNSUPPORTED,
                  "conv state length %lld implies a width-%lld convolution; "
                  "only width %d is supported (length = Q + 2)",
                  (long long)Lc, (long long)(Lc - Q + 2), kda::kConvWidth);
    if (!shape_is(a->conv_weight, C3, kda::kConvWidth))
      return fail(KDA_E_SHAPE, "conv_weight must be [%lld, %d]",
                  (long long)C3, kda::kConvWidth);
    if (a->conv_weight.dtype != KDA_F32 && a->conv_weight.dtype != act)
      return fail(KDA_E_DTYPE,
                  "conv_weight must be float32 or the activation dtype");
  }

  // Capacity (ops page: more tokens than the window allows is an error).
  if (T > int64_t(a->batch) * Q)
    return fail(KDA_E_CAPACITY,
                "KDA RecoverSSM speculative decode input exceeds its "
                "activation capacity (%lld tokens > %d x %lld)",
                (long long)T, a->batch, (long long)Q);
  if (int64_t(a->batch) * H > 0x7fffffff || T > 0x7fffffff)
    return fail(KDA_E_CAPACITY, "batch * heads or tokens exceed 2^31");

  // Static tensors: 16-byte starts (kernels page `_check_layouts`).
  const kda_tensor* statics[] = {&a->state, &a->A_log, &a->dt_bias,
                                 &a->correction, &a->key_gate, &cs, &cw};
  const char* snames[] = {"state", "A_log", "dt_bias", "correction",
                          "key_gate", "conv_state", "conv_weight"};
  for (int i = 0; i < 7; ++i)
    if (!aligned(statics[i]->data, 16))
      return fail(KDA_E_LAYOUT,
                  "KDA RecoverSSM: %s must start on a 16-byte boundary",
                  snames[i]);
  const int ek = elem_size(a->key_gate.dtype);
  for (int i = 0; i < 3; ++i)
    if ((a->correction.stride[i] * 4) % 16 != 0 ||
        (a->key_gate.stride[i] * ek) % 16 != 0)
      return fail(KDA_E_LAYOUT,
                  "record slot, head and position strides must be "
                  "multiples of 16 bytes");

  // Per-step tensors: not launched when misaligned (the caller may fall
  // back, as the kernels page's verify returns False).
  const int ea = elem_size(act), eo = elem_size(a->out.dtype);
  if (!aligned(a->mixed_qkv.data, 16) || !aligned(a->raw_gate.data, 16) ||
      !aligned(a->out.data, 16) ||
      (a->mixed_qkv.stride[0] * ea) % 16 != 0 ||
      (a->raw_gate.stride[0] * ea) % 16 != 0 ||
      (a->out.stride[0] * eo) % 16 != 0)
    return fail(KDA_E_UNALIGNED,
                "an activation or output row does not start on a 16-byte "
                "boundary");
  if (!aligned(a->raw_beta.data, ea))
    return fail(KDA_E_UNALIGNED, "raw_beta is not element aligned");

  // Metadata.
  if (a->items_per_ticket < 0)
    return fail(KDA_E_ARG, "items_per_ticket is negative");
  if (a->max_workgroups < 0)
    return fail(KDA_E_ARG, "max_workgroups is negative");
  if (a->schedule < KDA_SCHEDULE_DEFAULT || a->schedule > KDA_SCHEDULE_V_TILES)
    return fail(KDA_E_ARG, "unknown schedule %d", a->schedule);
  if (a->work_counter_len < 0)
    return fail(KDA_E_ARG, "work_counter_len is negative");
  if (a->v_tiles != 0 && a->v_tiles != 2 && a->v_tiles != 4 &&
      a->v_tiles != 8)
    return fail(KDA_E_ARG, "v_tiles must be 0, 2, 4 or 8 (got %d)",
                a->v_tiles);
  if (a->batch > 0) {
    if (!a->query_start_loc || !a->state_indices ||
        (conv && !a->num_accepted_tokens))
      return fail(KDA_E_ARG,
                  "query_start_loc, state_indices and num_accepted_tokens "
                  "are required");
    if (!a->work_counter && scratch_len == 0 &&
        a->schedule == KDA_SCHEDULE_TICKETS)
      return fail(KDA_E_ARG, "the ticket schedule needs a work_counter");
    if (a->pending_lens && a->batch > 65535)
      return fail(KDA_E_UNSUPPORTED,
                  "the deferred flush runs one workgroup per item and "
                  "supports at most 65535 requests");
    const void* ptrs[] = {a->query_start_loc, a->state_indices,
                          a->num_accepted_tokens, a->record_rows,
                          scratch_len > 0 ? nullptr : a->work_counter,
                          a->pending_lens};
    for (const void* q : ptrs)
      if (q && !aligned(q, 4))
        return fail(KDA_E_UNALIGNED, "metadata pointers must be 4-byte "
                                     "aligned");
  }

  // Every stride and every in-item offset the kernel forms must fit in 32
  // bits (slot and row strides are applied in 64-bit arithmetic).
  const int64_t i32max = 0x7fffffff;
  const int64_t strides[] = {
      a->mixed_qkv.stride[0], a->raw_gate.stride[0], a->raw_beta.stride[0],
      S.stride[0], a->correction.stride[0], a->correction.stride[1],
      a->correction.stride[2], a->key_gate.stride[0], a->key_gate.stride[1],
      a->key_gate.stride[2], a->out.stride[0], cs.stride[0], cs.stride[1],
      cs.stride[2], cw.stride[0], cw.stride[1]};
  for (int64_t st : strides)
    if (st < 0 || st > i32max)
      return fail(KDA_E_LAYOUT, "a tensor stride is negative or exceeds 2^31");
  const int64_t s_chan = a->conv_dim_first ? cs.stride[1] : cs.stride[2];
  const int64_t s_tok = a->conv_dim_first ? cs.stride[2] : cs.stride[1];
  if (C3 * s_chan + Lc * s_tok > i32max || C3 * cw.stride[0] > i32max ||
      Q * (a->mixed_qkv.stride[0] + a->raw_gate.stride[0] +
           a->raw_beta.stride[0] + a->out.stride[0]) > i32max ||
      Q * (a->correction.stride[2] + a->key_gate.stride[2]) + 2 * D >
          i32max)
    return fail(KDA_E_LAYOUT, "per-request offsets exceed 2^31 elements");
  // The out, correction and conv-tap accesses form their in-item offsets
  // in BYTES as unsigned 32-bit values from a wave-uniform base: bound
  // those byte offsets too (2^31, as the element offsets above).
  const int ew = conv ? elem_size(cw.dtype) : 0;
  if ((Q * a->out.stride[0] + D) * eo > i32max ||
      (Q * a->correction.stride[2] + D) * 4 > i32max ||
      (C3 * cw.stride[0] + kda::kConvWidth * cw.stride[1]) * ew > i32max)
    return fail(KDA_E_LAYOUT, "per-request byte offsets exceed 2^31");

  kda::VerifyParams& p = plan->p;
  p = kda::VerifyParams{};
  p.mixed_qkv = a->mixed_qkv.data;
  p.s_x = int32_t(a->mixed_qkv.stride[0]);
  p.raw_gate = a->raw_gate.data;
  p.s_g = int32_t(a->raw_gate.stride[0]);
  p.raw_beta = a->raw_beta.data;
  p.s_beta = int32_t(a->raw_beta.stride[0]);
  p.A_log = static_cast<const float*>(a->A_log.data);
  p.dt_bias = static_cast<const float*>(dtb.data);
  p.state = static_cast<const float*>(S.data);
  p.s_slot = int32_t(S.stride[0]);
  p.correction = static_cast<float*>(a->correction.data);
  p.s_c_row = int32_t(a->correction.stride[0]);
  p.s_c_head = int32_t(a->correction.stride[1]);
  p.s_c_pos = int32_t(a->correction.stride[2]);
  p.key_gate = a->key_gate.data;
  p.s_kg_row = int32_t(a->key_gate.stride[0]);
  p.s_kg_head = int32_t(a->key_gate.stride[1]);
  p.s_kg_pos = int32_t(a->key_gate.stride[2]);
  p.out = a->out.data;
  p.s_out = int32_t(a->out.stride[0]);
  p.conv_state = cs.data;
  p.s_cs_slot = int32_t(cs.stride[0]);
  p.s_cs_chan = int32_t(s_chan);
  p.s_cs_tok = int32_t(s_tok);
  p.conv_weight = cw.data;
  p.s_w_chan = int32_t(cw.stride[0]);
  p.s_w_tap = int32_t(cw.stride[1]);
  p.qsl = a->query_start_loc;
  p.slots = a->state_indices;
  p.accepted = conv ? a->num_accepted_tokens : a->state_indices;
  p.record_rows = a->record_rows;
  p.pending = a->pending_lens;
  p.counter = scratch_len > 0 ? nullptr : a->work_counter;
  p.B = a->batch;
  p.H = int32_t(H);
  p.Q = int32_t(Q);
  p.N = N > i32max ? int32_t(i32max) : int32_t(N);
  p.R = R > i32max ? int32_t(i32max) : int32_t(R);
  p.T = int32_t(T);
  p.null_id = a->null_block_id;
  p.flags = (a->out.dtype == KDA_BF16 ? kda::kOutBf16 : 0) |
            (a->key_gate.dtype == KDA_BF16 ? kda::kKgBf16 : 0) |
            (conv && cw.dtype == KDA_BF16 ? kda::kWBf16 : 0) |
            (conv ? 0 : kda::kNoConv) |
            (a->use_lower_bound ? kda::kLowerBound : 0);
  if (conv && a->conv_dim_first && s_tok == 1 &&
      (Q == 4 || Q == 8 || Q == 16) &&
      (Lc * ea) % 4 == 0 && (s_chan * ea) % 4 == 0 &&
      (cs.stride[0] * ea) % 4 == 0)
    p.flags |= kda::kConvRow;
  if (conv && cw.stride[1] == 1 && cw.stride[0] == kda::kConvWidth &&
      aligned(cw.data, uintptr_t(kda::kConvWidth) * elem_size(cw.dtype)))
    p.flags |= kda::kWRow;
  p.lb = a->lower_bound;
  p.n_items = int32_t(int64_t(a->batch) * H);
  p.per_ticket = a->items_per_ticket;

  // V-tiles: possible for head dims 64 and 128 and windows up to 8 without
  // the deferred flush; the fused conv needs one arrival counter per item.
  const int64_t counter_len =
      scratch_len > 0 ? scratch_len
      : a->work_counter == nullptr
          ? 0
          : (a->work_counter_len > 0 ? a->work_counter_len : 1);
  const int64_t items = int64_t(a->batch) * H;
  const bool vt_shape = (D == 64 || D == 128) && Q <= 8 &&
                        a->pending_lens == nullptr;
  const bool vt_counter = !conv || counter_len >= 1 + items;
  int schedule = a->schedule;
  int vt = a->v_tiles;
  if (schedule == KDA_SCHEDULE_V_TILES) {
    if (!vt_shape)
      return fail(KDA_E_UNSUPPORTED,
                  "the V-tile schedule supports head dims 64 and 128, "
                  "windows up to 8 and no pending_lens");
    if (!vt_counter && scratch_len > 0)
      return fail(KDA_E_CAPACITY,
                  "the allocation-free verify's scratch holds %lld "
                  "counters; V-tiles of %lld (request, head) items need "
                  "%lld",
                  (long long)scratch_len, (long long)items,
                  (long long)(1 + items));
    if (!vt_counter)
      return fail(KDA_E_ARG,
                  "the V-tile schedule of the fused conv verify needs a "
                  "work_counter of 1 + batch * heads = %lld elements",
                  (long long)(1 + items));
    if (vt == 0) vt = default_vtiles(items);
  }
  // The default schedule never takes V-tiles: measured on MI355X they are
  // not faster than whole items at any batch (one request: 6.9 us per
  // verify whole, 7.0 / 7.1 / 9.0 us with 2 / 4 / 8 tiles; 64 ragged
  // requests: 33.3 us whole, 34.7 / 43.8 / 68.6 us).
  // The verify of a small batch is bound by the latency of its phases,
  // which splitting the rows does not shorten.
  if (schedule == KDA_SCHEDULE_V_TILES && items * vt > 0x7fffffff)
    return fail(KDA_E_CAPACITY, "batch * heads * v_tiles exceeds 2^31");
  p.v_tiles = schedule == KDA_SCHEDULE_V_TILES ? vt : 0;
  plan->D = int(D);
  plan->act_bf16 = act == KDA_BF16;
  // No tokens is a no-op, except for the deferred flush: requests with an
  // empty window still fold their pending positions.
  plan->noop = a->batch == 0 || (T == 0 && a->pending_lens == nullptr);
  plan->grid = a->max_workgroups;
  plan->schedule = schedule;
  return KDA_OK;
}

struct CommitPlan {
  kda::CommitParams p;
  int D = 0;
  bool noop = false;
};

int plan_commit(const kda_commit_args* a, CommitPlan* plan) {
  if (a == nullptr) return fail(KDA_E_ARG, "commit arguments are NULL");
  if (a->num_layers < 1)
    return fail(KDA_E_ARG, "KDA RecoverSSM commit requires at least one "
                           "layer");
  if (a->batch < 0) return fail(KDA_E_ARG, "batch is negative");
  const int64_t H = a->num_heads, D = a->head_dim, Q = a->spec_query_len;
  if (H < 1) return fail(KDA_E_SHAPE, "num_heads must be positive");
  if (!supported_head_dim(D))
    return fail(KDA_E_UNSUPPORTED,
                "head dim %lld is not supported (16, 32, 64 or 128)",
                (long long)D);
  if (Q < 1 || Q > kda::kMaxWindow)
    return fail(KDA_E_UNSUPPORTED,
                "KDA RecoverSSM commit supports windows of 1 to %d",
                kda::kMaxWindow);
  if (a->num_slots < 1 || a->num_record_rows < 1)
    return fail(KDA_E_SHAPE, "the state pool and records need rows");
  if (!a->state_base_addrs || !a->state_block_strides ||
      !a->correction_base_addrs || !a->correction_block_strides ||
      !a->key_gate_base_addrs || !a->key_gate_block_strides)
    return fail(KDA_E_ARG, "the per-layer address tables are required");
  if (!a->A_log || !a->dt_bias || !a->use_lower_bound || !a->lower_bound)
    return fail(KDA_E_ARG, "the stacked gate parameters are required");
  if (a->batch > 0 && (!a->state_indices || !a->commit_lens))
    return fail(KDA_E_ARG, "state_indices and commit_lens are required");
  if (!a->boundary_state_indices != !a->boundary_recovery_lens)
    return fail(KDA_E_ARG,
                "KDA RecoverSSM align metadata is incomplete: boundary slots "
                "and boundary lengths go together");
  if (a->state_strides[0] != D * D || a->state_strides[1] != D)
    return fail(KDA_E_LAYOUT,
                "KDA RecoverSSM layers need contiguous checkpoint heads "
                "(strides %lld, %lld)",
                (long long)a->state_strides[0],
                (long long)a->state_strides[1]);
  const int ek = elem_size(a->key_gate_dtype);
  if (ek == 0) return fail(KDA_E_DTYPE, "key/gate dtype must be F32 or BF16");
  for (int i = 0; i < 2; ++i)
    if ((a->correction_strides[i] * 4) % 16 != 0 ||
        (a->key_gate_strides[i] * ek) % 16 != 0)
      return fail(KDA_E_LAYOUT,
                  "record head and position strides must be multiples of "
                  "16 bytes");
  if (int64_t(a->num_layers) * a->batch * H > 0x7fffffff)
    return fail(KDA_E_CAPACITY, "layers * batch * heads exceeds 2^31");
  if (a->host_tables) {
    const int64_t L = a->num_layers;
    const int64_t* t = a->host_tables;
    const int esz[3] = {4, 4, ek};
    const char* nm[3] = {"state", "correction", "key/gate"};
    for (int k = 0; k < 3; ++k)
      for (int64_t l = 0; l < L; ++l) {
        const int64_t base = t[(2 * k) * L + l];
        const int64_t bs = t[(2 * k + 1) * L + l];
        if (base == 0 || base % 16 != 0 || (bs * esz[k]) % 16 != 0)
          return fail(KDA_E_LAYOUT,
                      "layer %lld: %s view must start on a 16-byte boundary "
                      "with 16-byte aligned slots",
                      (long long)l, nm[k]);
      }
  }
  kda::CommitParams& p = plan->p;
  p = kda::CommitParams{};
  p.state_base = a->state_base_addrs;
  p.state_bs = a->state_block_strides;
  p.corr_base = a->correction_base_addrs;
  p.corr_bs = a->correction_block_strides;
  p.kg_base = a->key_gate_base_addrs;
  p.kg_bs = a->key_gate_block_strides;
  p.s_state_head = a->state_strides[0];
  p.s_c_head = a->correction_strides[0];
  p.s_c_pos = a->correction_strides[1];
  p.s_kg_head = a->key_gate_strides[0];
  p.s_kg_pos = a->key_gate_strides[1];
  p.A_log = a->A_log;
  p.s_A_l = a->A_log_strides[0];
  p.s_A_h = a->A_log_strides[1];
  p.dt_bias = a->dt_bias;
  p.s_dt_l = a->dt_bias_strides[0];
  p.s_dt_h = a->dt_bias_strides[1];
  p.s_dt_d = a->dt_bias_strides[2];
  p.use_lb = a->use_lower_bound;
  p.lb = a->lower_bound;
  p.slots = a->state_indices;
  p.commit_lens = a->commit_lens;
  p.final_slots = a->final_state_indices;
  p.record_rows = a->record_rows;
  p.bnd_slots = a->boundary_state_indices;
  p.bnd_lens = a->boundary_recovery_lens;
  p.L = a->num_layers;
  p.B = a->batch;
  p.H = int32_t(H);
  p.Q = int32_t(Q);
  p.null_id = a->null_block_id;
  p.N = a->num_slots;
  p.R = a->num_record_rows;
  p.kg_bf16 = a->key_gate_dtype == KDA_BF16;
  p.grid = a->max_workgroups;
  plan->D = int(D);
  plan->noop = a->batch == 0;
  return KDA_OK;
}

// Commit plan (ops page `KDARecoverSSMCommitContext.commit` checks: align
// arguments all or none, a block that covers one window, a 2-D table).
int plan_plan(const kda_plan_args* a, kda::PlanParams* p) {
  if (a == nullptr) return fail(KDA_E_ARG, "plan arguments are NULL");
  if (a->batch < 0) return fail(KDA_E_ARG, "batch is negative");
  if (a->spec_query_len < 1 || a->spec_query_len > kda::kMaxWindow)
    return fail(KDA_E_UNSUPPORTED,
                "KDA RecoverSSM supports windows of 1 to %d",
                kda::kMaxWindow);
  const bool align = a->block_table != nullptr;
  if (align != (a->num_computed_tokens != nullptr))
    return fail(KDA_E_ARG, "KDA RecoverSSM align metadata is incomplete");
  if (align) {
    if (a->mamba_block_size < a->spec_query_len)
      return fail(KDA_E_ARG,
                  "KDA RecoverSSM align block size must cover one "
                  "speculative window");
    if (a->block_table_width < 1)
      return fail(KDA_E_SHAPE, "the block table needs at least one column");
    if (a->block_table_strides[0] < 0 || a->block_table_strides[1] < 0)
      return fail(KDA_E_LAYOUT, "block table strides must be non-negative");
    if (!aligned(a->block_table, 4) || !aligned(a->num_computed_tokens, 4))
      return fail(KDA_E_UNALIGNED, "align metadata must be 4-byte aligned");
  }
  if (a->batch > 0) {
    if (!a->num_accepted_tokens || !a->state_indices || !a->query_start_loc)
      return fail(KDA_E_ARG,
                  "num_accepted_tokens, state_indices and query_start_loc "
                  "are required");
    if (!a->commit_lens || !a->final_state_indices ||
        !a->boundary_state_indices || !a->boundary_recovery_lens)
      return fail(KDA_E_ARG, "the four plan outputs are required");
    if (a->num_request_rows < 0 ||
        (!a->request_indices && a->num_request_rows < a->batch))
      return fail(KDA_E_ARG,
                  "KDA RecoverSSM request mapping is too short (%d rows for "
                  "%d requests)", a->num_request_rows, a->batch);
    const void* ptrs[] = {a->num_accepted_tokens, a->request_indices,
                          a->state_indices, a->query_start_loc,
                          a->commit_lens, a->final_state_indices,
                          a->boundary_state_indices,
                          a->boundary_recovery_lens};
    for (const void* q : ptrs)
      if (q && !aligned(q, 4))
        return fail(KDA_E_UNALIGNED, "plan arrays must be 4-byte aligned");
  }
  *p = kda::PlanParams{};
  p->accepted = a->num_accepted_tokens;
  p->req_idx = a->request_indices;
  p->slots = a->state_indices;
  p->qsl = a->query_start_loc;
  p->table = a->block_table;
  p->s_tab_row = a->block_table_strides[0];
  p->s_tab_col = a->block_table_strides[1];
  p->computed = a->num_computed_tokens;
  p->lens = a->commit_lens;
  p->final_slots = a->final_state_indices;
  p->bnd_slots = a->boundary_state_indices;
  p->bnd_lens = a->boundary_recovery_lens;
  p->B = a->batch;
  p->Q = a->spec_query_len;
  p->null_id = a->null_block_id;
  p->block = align ? a->mamba_block_size : 1;
  p->rows = a->request_indices ? a->num_request_rows : a->batch;
  p->width = align ? a->block_table_width : 1;
  return KDA_OK;
}

// Conv compaction (ops page `KDARecoverSSMCommitContext.create`: matching
// conv states in every layer, history = length - Q + 1).
int plan_compact(const kda_compact_args* a, kda::CompactParams* p,
                 int* elem_bytes) {
  if (a == nullptr) return fail(KDA_E_ARG, "compaction arguments are NULL");
  if (a->batch < 0) return fail(KDA_E_ARG, "batch is negative");
  if (a->num_layers < 1)
    return fail(KDA_E_ARG, "KDA RecoverSSM commit requires at least one "
                           "layer");
  if (a->spec_query_len < 1 || a->spec_query_len > kda::kMaxWindow)
    return fail(KDA_E_UNSUPPORTED,
                "KDA RecoverSSM supports windows of 1 to %d",
                kda::kMaxWindow);
  if (a->num_slots < 1 || a->conv_dim < 1 || a->conv_dim > 0x7fffffff)
    return fail(KDA_E_SHAPE, "the conv state pool needs slots and channels");
  const int e = elem_size(a->conv_dtype);
  if (e == 0) return fail(KDA_E_DTYPE, "conv state dtype must be F32 or BF16");
  if (!a->conv_tables)
    return fail(KDA_E_ARG, "the per-layer conv tables are required");
  if (!a->boundary_state_indices != !a->boundary_recovery_lens)
    return fail(KDA_E_ARG, "KDA RecoverSSM align metadata is incomplete");
  if (a->batch > 0 && (!a->state_indices || !a->commit_lens))
    return fail(KDA_E_ARG, "state_indices and commit_lens are required");
  if (a->batch > 65535 || a->num_layers > 65535)
    return fail(KDA_E_UNSUPPORTED,
                "the compaction grid holds at most 65535 requests and layers");
  if (a->host_conv_tables) {
    const int64_t L = a->num_layers;
    const int64_t* t = a->host_conv_tables;
    const int64_t Lc = a->spec_query_len + kda::kConvWidth - 2;
    for (int64_t l = 0; l < L; ++l) {
      const int64_t base = t[l], ss = t[L + l], sc = t[2 * L + l],
                    st = t[3 * L + l];
      if (base == 0 || base % e != 0)
        return fail(KDA_E_LAYOUT, "layer %lld: conv state base is not "
                                  "element aligned", (long long)l);
      if (ss < 0 || sc < 0 || st < 0)
        return fail(KDA_E_LAYOUT, "layer %lld: negative conv state stride",
                    (long long)l);
      // the last element every channel can touch stays inside its slot
      if ((a->conv_dim - 1) * sc + (Lc - 1) * st >= ss && a->num_slots > 1)
        return fail(KDA_E_LAYOUT, "layer %lld: conv state slots overlap",
                    (long long)l);
    }
  }
  *p = kda::CompactParams{};
  p->tables = a->conv_tables;
  p->slots = a->state_indices;
  p->commit_lens = a->commit_lens;
  p->final_slots = a->final_state_indices;
  p->bnd_slots = a->boundary_state_indices;
  p->bnd_lens = a->boundary_recovery_lens;
  p->L = a->num_layers;
  p->B = a->batch;
  p->Q = a->spec_query_len;
  p->null_id = a->null_block_id;
  p->N = a->num_slots;
  p->C = int32_t(a->conv_dim);
  *elem_bytes = e;
  return KDA_OK;
}

// Fused commit step: the three argument blocks must describe one batch
// exactly as they would for the three separate calls (the commit and the
// compaction read the plan's output arrays).
bool reads_plan(const int32_t* si, const int32_t* lens, const int32_t* fin,
                const int32_t* bnd, const int32_t* blen,
                const kda_plan_args* pl) {
  const bool align = pl->block_table != nullptr;
  return si == pl->state_indices && lens == pl->commit_lens &&
         fin == pl->final_state_indices &&
         (align ? (bnd == pl->boundary_state_indices &&
                   blen == pl->boundary_recovery_lens)
                : (bnd == nullptr && blen == nullptr));
}

int plan_step(const kda_commit_args* c, const kda_plan_args* pl,
              const kda_compact_args* cp, CommitPlan* plan) {
  if (c == nullptr || pl == nullptr)
    return fail(KDA_E_ARG, "the commit step needs commit and plan arguments");
  KDA_TRY(plan_commit(c, plan));
  kda::PlanParams pp;
  KDA_TRY(plan_plan(pl, &pp));
  if (pl->batch != c->batch || pl->spec_query_len != c->spec_query_len ||
      pl->null_block_id != c->null_block_id)
    return fail(KDA_E_ARG, "commit step: the plan and the commit describe "
                           "different batches");
  if (c->batch > 0 &&
      !reads_plan(c->state_indices, c->commit_lens, c->final_state_indices,
                  c->boundary_state_indices, c->boundary_recovery_lens, pl))
    return fail(KDA_E_ARG,
                "commit step: the commit must take the plan's state_indices "
                "and its output arrays (boundary pair only in align mode)");
  plan->p.step = 1;
  plan->p.plan = pp;
  if (cp != nullptr) {
    kda::CompactParams q;
    int e = 0;
    KDA_TRY(plan_compact(cp, &q, &e));
    if (cp->batch != c->batch || cp->num_layers != c->num_layers ||
        cp->spec_query_len != c->spec_query_len ||
        cp->null_block_id != c->null_block_id ||
        cp->num_slots != c->num_slots ||
        cp->conv_dim != 3 * int64_t(c->num_heads) * c->head_dim)
      return fail(KDA_E_ARG,
                  "commit step: the compaction and the commit describe "
                  "different batches, layers or pools (conv_dim must be "
                  "3 * heads * head_dim)");
    if (c->batch > 0 &&
        !reads_plan(cp->state_indices, cp->commit_lens,
                    cp->final_state_indices, cp->boundary_state_indices,
                    cp->boundary_recovery_lens, pl))
      return fail(KDA_E_ARG,
                  "commit step: the compaction must take the plan's "
                  "state_indices and its output arrays (boundary pair only "
                  "in align mode)");
    plan->p.conv_tables = cp->conv_tables;
    plan->p.conv_elem = e;
  }
  return KDA_OK;
}

int device_status(int hip_rc, const char* what) {
  if (hip_rc == 0) return KDA_OK;
  return fail(KDA_E_DEVICE, "%s: HIP error %d (%s)", what, hip_rc,
              hipGetErrorString(hipError_t(hip_rc)));
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_last_error(void) { return g_err.c_str(); }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_E_SHAPE: return "KDA_E_SHAPE";
    case KDA_E_DTYPE: return "KDA_E_DTYPE";
    case KDA_E_LAYOUT: return "KDA_E_LAYOUT";
    case KDA_E_UNALIGNED: return "KDA_E_UNALIGNED";
    case KDA_E_UNSUPPORTED: return "KDA_E_UNSUPPORTED";
    case KDA_E_CAPACITY: return "KDA_E_CAPACITY";
    case KDA_E_DEVICE: return "KDA_E_DEVICE";
    case KDA_E_ARG: return "KDA_E_ARG";
    default: return "KDA_E_UNKNOWN";
  }
}

int kda_check_verify(const kda_verify_args* args) {
  g_err.clear();
  VerifyPlan plan;
  return plan_verify(args, &plan, true);
}

int kda_check_verify_qkv(const kda_verify_args* args) {
  g_err.clear();
  VerifyPlan plan;
  return plan_verify(args, &plan, false);
}

int kda_recoverssm_verify_qkv(const kda_verify_args* args, void* stream) {
  g_err.clear();
  VerifyPlan plan;
  KDA_TRY(plan_verify(args, &plan, false));
  if (plan.noop) return KDA_OK;
  return device_status(
      kda::launch_verify(plan.p, plan.D, plan.act_bf16, plan.schedule,
                         plan.grid, static_cast<hipStream_t>(stream)),
      "kda_recoverssm_verify_qkv launch");
}

int kda_conv_update_verify(const kda_verify_args* args, void* stream) {
  g_err.clear();
  VerifyPlan plan;
  KDA_TRY(plan_verify(args, &plan, true));
  if (plan.noop) return KDA_OK;
  return device_status(
      kda::launch_verify(plan.p, plan.D, plan.act_bf16, plan.schedule,
                         plan.grid,
                         static_cast<hipStream_t>(stream)),
      "kda_conv_update_verify launch");
}

int kda_conv_update_verify_noalloc(const kda_verify_args* args,
                                   void* stream) {
  g_err.clear();
  // Every host check first (with the scratch standing in for the counter
  // array), so that a batch the scratch cannot serve is refused before any
  // device call.
  VerifyPlan plan;
  KDA_TRY(plan_verify(args, &plan, true, kda::kScratchCounters));
  if (plan.noop) return KDA_OK;
  int32_t* counters = nullptr;
  const int e = kda::scratch_counters(static_cast<hipStream_t>(stream),
                                      &counters);
  if (e != 0)
    return device_status(e, "kda_conv_update_verify_noalloc scratch");
  plan.p.counter = counters;
  return device_status(
      kda::launch_verify(plan.p, plan.D, plan.act_bf16, plan.schedule,
                         plan.grid, static_cast<hipStream_t>(stream)),
      "kda_conv_update_verify_noalloc launch");
}

int kda_check_commit(const kda_commit_args* args) {
  g_err.clear();
  CommitPlan plan;
  return plan_commit(args, &plan);
}

int kda_recoverssm_commit(const kda_commit_args* args, void* stream) {
  g_err.clear();
  CommitPlan plan;
  KDA_TRY(plan_commit(args, &plan));
  if (plan.noop) return KDA_OK;
  return device_status(
      kda::launch_commit(plan.p, plan.D, static_cast<hipStream_t>(stream)),
      "kda_recoverssm_commit launch");
}

int kda_check_commit_plan(const kda_plan_args* args) {
  g_err.clear();
  kda::PlanParams p;
  return plan_plan(args, &p);
}

int kda_commit_plan(const kda_plan_args* args, void* stream) {
  g_err.clear();
  kda::PlanParams p;
  KDA_TRY(plan_plan(args, &p));
  if (p.B == 0) return KDA_OK;
  return device_status(
      kda::launch_commit_plan(p, static_cast<hipStream_t>(stream)),
      "kda_commit_plan launch");
}

int kda_check_compact_conv(const kda_compact_args* args) {
  g_err.clear();
  kda::CompactParams p;
  int e = 0;
  return plan_compact(args, &p, &e);
}

int kda_compact_conv_state(const kda_compact_args* args, void* stream) {
  g_err.clear();
  kda::CompactParams p;
  int e = 0;
  KDA_TRY(plan_compact(args, &p, &e));
  if (p.B == 0) return KDA_OK;
  return device_status(
      kda::launch_compact(p, e, static_cast<hipStream_t>(stream)),
      "kda_compact_conv_state launch");
}

int kda_check_commit_step(const kda_commit_args* commit,
                          const kda_plan_args* plan,
                          const kda_compact_args* compact) {
  g_err.clear();
  CommitPlan cp;
  return plan_step(commit, plan, compact, &cp);
}

int kda_recoverssm_commit_step(const kda_commit_args* commit,
                               const kda_plan_args* plan,
                               const kda_compact_args* compact,
                               void* stream) {
  g_err.clear();
  CommitPlan cp;
  KDA_TRY(plan_step(commit, plan, compact, &cp));
  if (cp.noop) return KDA_OK;
  return device_status(
      kda::launch_commit(cp.p, cp.D, static_cast<hipStream_t>(stream)),
      "kda_recoverssm_commit_step launch");
}

int kda_set_launch_events(void* start_event, void* stop_event,
                          int32_t launches, int32_t* pending) {
  g_err.clear();
  if (launches < 0)
    return fail(KDA_E_ARG, "kda_set_launch_events needs launches >= 0");
  kda::LaunchTiming& t = kda::launch_timing();
  if (pending) *pending = t.remaining;
  t.start = launches > 0 ? static_cast<hipEvent_t>(start_event) : nullptr;
  t.stop = launches > 0 ? static_cast<hipEvent_t>(stop_event) : nullptr;
  t.remaining = launches;
  return KDA_OK;
}

int kda_reset_counter(int32_t* counter, int32_t n, void* stream) {
  g_err.clear();
  if (counter == nullptr || n < 1)
    return fail(KDA_E_ARG, "kda_reset_counter needs a counter and n >= 1");
  return device_status(kda::launch_reset_counter(
                           counter, n, static_cast<hipStream_t>(stream)),
                       "kda_reset_counter launch");
}

}  // extern "C"
