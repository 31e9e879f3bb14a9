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
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kCompactThreads = 256;

__global__ void __launch_bounds__(kPlanThreads)
    kda_commit_plan_kernel(PlanParams p) {
  const int b = blockIdx.x * kPlanThreads + threadIdx.x;
  if (b >= p.B) return;
  const int slot = p.slots[b];
  const int row = p.req_idx ? p.req_idx[b] : b;
  const int q = min(max(p.qsl[b + 1] - p.qsl[b], 0), p.Q);
  int n = 0;
  if (row >= 0 && row < p.rows && slot > p.null_id)
    n = min(max(p.accepted[row], 0), q);
  int final_slot = slot, bnd = p.null_id, blen = 0;
  if (p.table && n > 0) {
    const int64_t c = max(p.computed[row], 0);
    const int64_t last = (c + n) / p.block;    // block of the next token
    final_slot = last < p.width
                     ? p.table[row * p.s_tab_row + last * p.s_tab_col]
                     : p.null_id;
    const int64_t start = last * p.block;
    if (c < start && last - 1 < p.width) {     // the block before is full
      bnd = p.table[row * p.s_tab_row + (last - 1) * p.s_tab_col];
      blen = int(start - c);
    }
  }
  p.lens[b] = n;
  p.final_slots[b] = final_slot;
  p.bnd_slots[b] = bnd;
  p.bnd_lens[b] = blen;
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
  T* base = reinterpret_cast<T*>(p.tables[l]);
  const int64_t s_slot = p.tables[L + l];
  const int64_t s_ch = p.tables[2 * L + l];
  const int64_t s_tok = p.tables[3 * L + l];
  const T* src = base + slot * s_slot + ch * s_ch;
  T hn[kConvWidth - 1], hb[kConvWidth - 1];
#pragma unroll
  for (int i = 0; i < kConvWidth - 1; ++i) {
    hn[i] = src[(n - 1 + i) * s_tok];
    hb[i] = bs >= 0 ? src[(m - 1 + i) * s_tok] : T{};
  }
  if (bs >= 0) {
    T* dst = base + bs * s_slot + ch * s_ch;
#pragma unroll
    for (int i = 0; i < kConvWidth - 1; ++i) dst[i * s_tok] = hb[i];
  }
  T* dst = base + f * s_slot + ch * s_ch;
#pragma unroll
  for (int i = 0; i < kConvWidth - 1; ++i) dst[i * s_tok] = hn[i];
}

}  // namespace

int launch_commit_plan(const PlanParams& p, hipStream_t stream) {
  if (p.B <= 0) return 0;
  const int blocks = (p.B + kPlanThreads - 1) / kPlanThreads;
  hipLaunchKernelGGL(kda_commit_plan_kernel, dim3(blocks), dim3(kPlanThreads),
                     0, stream, p);
  return int(hipGetLastError());
}

int launch_compact(const CompactParams& p, int elem_bytes, hipStream_t stream) {
  if (p.B <= 0 || p.L <= 0 || p.C <= 0) return 0;
  if (p.B > 65535 || p.L > 65535) return int(hipErrorInvalidValue);
  const dim3 grid((p.C + kCompactThreads - 1) / kCompactThreads, p.B, p.L);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(kda_compact_conv_kernel<uint16_t>, grid,
                       dim3(kCompactThreads), 0, stream, p);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(kda_compact_conv_kernel<uint32_t>, grid,
                       dim3(kCompactThreads), 0, stream, p);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace kda
