// Commit plan and conv-state compaction for gfx950: the two launches the ops
// page's `KDARecoverSSMCommitContext.commit` runs before the state commit
// (`_prepare_commit_plan_kernel`, `_compact_conv_state_kernel`; neither body
// is on the pages, the semantics implemented are the ones the public header
// states).
//
// Both are tiny integer / copy kernels: the plan touches a few words per
// request, the compaction moves (W - 1) conv-state entries per channel, so
// neither needs LDS or wide tiles; the compaction's grid puts consecutive
// channels of one (request, layer) in one workgroup so the channel-strided
// accesses of a dim-first state fall in neighbouring rows.
#include "kda_step.hpp"

namespace kda {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kCompactThreads = 256;

__global__ void __launch_bounds__(kPlanThreads)
    kda_commit_plan_kernel(PlanParams p) {
  const int b = blockIdx.x * kPlanThreads + threadIdx.x;
  if (b >= p.B) return;
  store_plan(p, b, plan_request(p, b));
}

template <class T>
__global__ void __launch_bounds__(kCompactThreads)
    kda_compact_conv_kernel(CompactParams p) {
  const int ch = blockIdx.x * kCompactThreads + threadIdx.x;
  const int b = blockIdx.y, l = blockIdx.z;
  const int slot = p.slots[b];
  if (slot <= p.null_id || slot < 0 || slot >= p.N) return;
  const int n = min(max(p.commit_lens[b], 0), p.Q);
  if (n == 0) return;
  const int f = p.final_slots ? p.final_slots[b] : slot;
  if (f <= p.null_id || f < 0 || f >= p.N) return;
  int bs = -1, m = 0;
  if (p.bnd_slots) {
    bs = p.bnd_slots[b];
    m = min(max(p.bnd_lens[b], 0), n);
    if (bs <= p.null_id || bs < 0 || bs >= p.N || m < 1) bs = -1;
  }
  if (ch >= p.C) return;
  const int64_t L = p.L;
  T* base = global_addr<T>(p.tables[l]);
  const int64_t s_slot = p.tables[L + l];
  const int64_t s_ch = p.tables[2 * L + l];
  const int64_t s_tok = p.tables[3 * L + l];
  const T* src = base + slot * s_slot + ch * s_ch;
  // everything is read before anything is written
  const ConvHistory<T> hn = load_history(src, s_tok, n);
  ConvHistory<T> hb{};
  if (bs >= 0) hb = load_history(src, s_tok, m);
  if (bs >= 0) store_history(base + bs * s_slot + ch * s_ch, s_tok, hb);
  store_history(base + f * s_slot + ch * s_ch, s_tok, hn);
}

}  // namespace

int launch_commit_plan(const PlanParams& p, hipStream_t stream) {
  if (p.B <= 0) return 0;
  const int blocks = (p.B + kPlanThreads - 1) / kPlanThreads;
  launch_kernel(kda_commit_plan_kernel, dim3(blocks), dim3(kPlanThreads),
                0, stream, p);
  return int(hipGetLastError());
}

int launch_compact(const CompactParams& p, int elem_bytes, hipStream_t stream) {
  if (p.B <= 0 || p.L <= 0 || p.C <= 0) return 0;
  if (p.B > 65535 || p.L > 65535) return int(hipErrorInvalidValue);
  const dim3 grid((p.C + kCompactThreads - 1) / kCompactThreads, p.B, p.L);
  if (elem_bytes == 2)
    launch_kernel(kda_compact_conv_kernel<uint16_t>, grid,
                  dim3(kCompactThreads), 0, stream, p);
  else if (elem_bytes == 4)
    launch_kernel(kda_compact_conv_kernel<uint32_t>, grid,
                  dim3(kCompactThreads), 0, stream, p);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace kda
