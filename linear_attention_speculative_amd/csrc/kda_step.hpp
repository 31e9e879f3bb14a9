// Device pieces shared by the commit plan and conv compaction kernels and by
// the fused commit step (the commit kernel doing both inline): the plan of
// one request and the copy of one channel's conv history.  Semantics are the
// ones the public header states for kda_commit_plan and
// kda_compact_conv_state.
#pragma once

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

struct RequestPlan {
  int n;       // positions to commit, in [0, q_b]
  int final_slot;
  int bnd;     // boundary slot, or the null id
  int blen;    // boundary length (0 without a boundary)
};

// Plan of request b: commit length from the accepted count of its row,
// final slot and (with a block table) the boundary block and its length.
__device__ __forceinline__ RequestPlan plan_request(const PlanParams& p,
                                                    int b) {
  const int slot = p.slots[b];
  const int row = p.req_idx ? p.req_idx[b] : b;
  const int q = min(max(p.qsl[b + 1] - p.qsl[b], 0), p.Q);
  RequestPlan r{0, slot, p.null_id, 0};
  if (row >= 0 && row < p.rows && slot > p.null_id)
    r.n = min(max(p.accepted[row], 0), q);
  if (p.table && r.n > 0) {
    const int64_t c = max(p.computed[row], 0);
    const int64_t last = (c + r.n) / p.block;  // block of the next token
    r.final_slot = last < p.width
                       ? p.table[row * p.s_tab_row + last * p.s_tab_col]
                       : p.null_id;
    const int64_t start = last * p.block;
    if (c < start && last - 1 < p.width) {     // the block before is full
      r.bnd = p.table[row * p.s_tab_row + (last - 1) * p.s_tab_col];
      r.blen = int(start - c);
    }
  }
  return r;
}

__device__ __forceinline__ void store_plan(const PlanParams& p, int b,
                                           const RequestPlan& r) {
  p.lens[b] = r.n;
  p.final_slots[b] = r.final_slot;
  p.bnd_slots[b] = r.bnd;
  p.bnd_lens[b] = r.blen;
}

// The W - 1 history entries of one channel that follow `k` committed
// positions of the verify's rolled row: entries [k - 1, k - 1 + W - 1).
template <class T>
struct ConvHistory {
  T v[kConvWidth - 1];
};

template <class T>
__device__ __forceinline__ ConvHistory<T> load_history(const T* row,
                                                       int64_t s_tok, int k) {
  ConvHistory<T> h;
#pragma unroll
  for (int i = 0; i < kConvWidth - 1; ++i) h.v[i] = row[(k - 1 + i) * s_tok];
  return h;
}

// Written to entries [0, W - 1) of a slot's row (read with accepted count 1
// by the next verify).
template <class T>
__device__ __forceinline__ void store_history(T* row, int64_t s_tok,
                                              const ConvHistory<T>& h) {
#pragma unroll
  for (int i = 0; i < kConvWidth - 1; ++i) row[i * s_tok] = h.v[i];
}

}  // namespace kda
