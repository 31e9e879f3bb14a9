// Internal launch descriptors shared by the host library and the HIP
// kernels.  Not part of the public ABI (see include/kda_recoverssm.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Timing armed by kda_set_launch_events on the calling thread: the next
// `remaining` launches made through launch_kernel are dispatched with
// hipExtLaunchKernel, `start` on the first and `stop` on the last.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  int remaining = 0;
};
LaunchTiming& launch_timing();

// Launch of a verify, commit, plan or compaction kernel.
template <typename... Args, typename F>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem,
                          hipStream_t stream, Args... args) {
  LaunchTiming& t = launch_timing();
  if (t.remaining <= 0) {
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
    return;
  }
  hipEvent_t start = t.start;
  hipEvent_t stop = t.remaining == 1 ? t.stop : nullptr;
  t.start = nullptr;
  if (--t.remaining == 0) t.stop = nullptr;
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start, stop, 0,
                        args...);
}

constexpr int kConvWidth = 4;   // taps of the short convolution
constexpr int kMaxWindow = 16;  // largest draft window Q supported

// Everything the verify kernel needs.  Strides are in elements and fit in
// 32 bits (checked on the host); keeping them narrow keeps the kernel's
// wave-uniform state inside the scalar register file.
struct VerifyParams {
  const void* mixed_qkv;    // [T, 3HD]
  const void* raw_gate;     // [T, HD]
  const void* raw_beta;     // [T, H]
  const float* A_log;       // [H]
  const float* dt_bias;     // [H, D]
  const float* state;       // [N, H, D, D]
  float* correction;        // [R, H, Q, D]
  void* key_gate;           // [R, H, Q, 2D]
  void* out;                // [T, HD]
  void* conv_state;         // [N, 3HD, Lc] / [N, Lc, 3HD]
  const void* conv_weight;  // [3HD, W]
  const int32_t* qsl;
  const int32_t* slots;
  const int32_t* accepted;
  const int32_t* record_rows;  // may be null
  const int32_t* pending;      // may be null: positions to flush first
  int32_t* counter;
  int32_t s_x, s_g, s_beta, s_slot;
  int32_t s_c_row, s_c_head, s_c_pos;
  int32_t s_kg_row, s_kg_head, s_kg_pos;
  int32_t s_out;
  int32_t s_cs_slot, s_cs_chan, s_cs_tok;
  int32_t s_w_chan, s_w_tap;
  int32_t B, H, Q, N, R, T, null_id;
  int32_t flags;            // kOutBf16 | kKgBf16 | kWBf16 | kLowerBound
  float lb;
  int32_t n_items;
  int32_t per_ticket;       // items claimed per ticket
  int32_t n_tickets;        // ceil(n_items / per_ticket)
  int32_t v_tiles;          // V-tile schedule: workgroups per item (2, 4, 8)
};

constexpr int32_t kOutBf16 = 1;
constexpr int32_t kKgBf16 = 2;
constexpr int32_t kWBf16 = 4;
constexpr int32_t kLowerBound = 8;
// dim-first conv state whose rows (Q + 2 elements, Q in {4, 8, 16}) are
// contiguous and 4-byte aligned: read and rolled a whole row at a time
constexpr int32_t kConvRow = 16;
// mixed_qkv already holds the convolved q | k | v: no conv, no roll
constexpr int32_t kNoConv = 64;
// each channel's four taps are contiguous and their row is aligned to its
// size (8 bytes in bf16, 16 in fp32): read with one load per channel
constexpr int32_t kWRow = 128;

// Commit plan of each request (one thread per request, or inline in the
// fused commit step).
struct PlanParams {
  const int32_t* accepted;   // per request row
  const int32_t* req_idx;    // [B] or null (row = b)
  const int32_t* slots;      // [B]
  const int32_t* qsl;        // [B + 1]
  const int32_t* table;      // align mode, or null
  int64_t s_tab_row, s_tab_col;
  const int32_t* computed;   // per request row (align mode)
  int32_t* lens;
  int32_t* final_slots;
  int32_t* bnd_slots;
  int32_t* bnd_lens;
  int32_t B, Q, null_id, block, rows, width;
};

struct CommitParams {
  const int64_t* state_base;  const int64_t* state_bs;
  const int64_t* corr_base;   const int64_t* corr_bs;
  const int64_t* kg_base;     const int64_t* kg_bs;
  int64_t s_state_head;
  int64_t s_c_head, s_c_pos;
  int64_t s_kg_head, s_kg_pos;
  const float* A_log;   int64_t s_A_l, s_A_h;
  const float* dt_bias; int64_t s_dt_l, s_dt_h, s_dt_d;
  const int32_t* use_lb;
  const float* lb;
  const int32_t* slots;
  const int32_t* commit_lens;
  const int32_t* final_slots;   // may be null
  const int32_t* record_rows;   // may be null
  const int32_t* bnd_slots;     // align mode (both given) or null
  const int32_t* bnd_lens;
  int32_t L, B, H, Q, null_id;
  int64_t N, R;
  int32_t kg_bf16;
  int32_t grid;   // <= 0: one workgroup per item; > 0: persistent, strided
  // Fused commit step: every item plans its request inline (commit_lens,
  // final_slots and bnd_* are then not read; the layer-0, head-0 item of a
  // request writes the plan's outputs) and, with conv tables, copies its
  // head's conv histories as the compaction does.
  int32_t step;
  int32_t conv_elem;            // bytes per conv-state element (2 or 4)
  const int64_t* conv_tables;   // [4][L] as CompactParams::tables, or null
  PlanParams plan;
};

// Conv-state compaction: one thread per (layer, request, channel).
struct CompactParams {
  const int64_t* tables;     // [4][L]: base, slot, channel, token strides
  const int32_t* slots;
  const int32_t* commit_lens;
  const int32_t* final_slots;  // may be null (in place)
  const int32_t* bnd_slots;    // may be null
  const int32_t* bnd_lens;
  int32_t L, B, Q, null_id;
  int64_t N;
  int32_t C;                 // channels
};

// Verify schedules (kda_schedule of the public header).
constexpr int kScheduleDefault = 0;
constexpr int kSchedulePerItem = 1;
constexpr int kScheduleTickets = 2;
constexpr int kScheduleVTiles = 3;

// Launchers (return a hipError_t as int).  `grid` <= 0: as many persistent
// workgroups as are resident at once.
int launch_verify(const VerifyParams& p, int D, bool act_bf16, int schedule,
                  int grid, hipStream_t stream);
// The verify launches of one head dim (16, 32, 64, 128), each defined in
// its own translation unit.
template <int D>
int launch_verify_dim(const VerifyParams& p, bool act_bf16, int schedule,
                      int grid, hipStream_t stream);
int launch_commit(const CommitParams& p, int D, hipStream_t stream);
int launch_commit_plan(const PlanParams& p, hipStream_t stream);
int launch_compact(const CompactParams& p, int elem_bytes, hipStream_t stream);
int launch_reset_counter(int32_t* counter, int n, hipStream_t stream);

// The allocation-free verify's counters: kScratchCounters int32 in a
// per-GPU array of the library (the ticket counter, then one arrival
// counter per (request, head)).  Sets *out to the current device's copy;
// the first call on a device looks its address up and clears it with a
// kernel on `stream`.
constexpr int kScratchCounters = 1 + 65536;
int scratch_counters(hipStream_t stream, int32_t** out);

}  // namespace kda
