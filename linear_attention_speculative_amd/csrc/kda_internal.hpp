// Internal launch descriptors shared by the host library and the HIP
// kernels.  Not part of the public ABI (see include/kda_recoverssm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kConvWidth = 4;   // taps of the short convolution
constexpr int kMaxWindow = 16;  // largest draft window Q supported

// Everything the verify kernel needs, with strides in elements.
struct VerifyParams {
  const void* mixed_qkv;  int64_t s_x;      // [T, 3HD] row stride
  const void* raw_gate;   int64_t s_g;      // [T, HD]
  const void* raw_beta;   int64_t s_beta;   // [T, H]
  const float* A_log;                        // [H]
  const float* dt_bias;                      // [H, D]
  const float* state;     int64_t s_slot;   // [N, H, D, D]
  float* correction;      int64_t s_c_row, s_c_head, s_c_pos;
  void* key_gate;         int64_t s_kg_row, s_kg_head, s_kg_pos;
  void* out;              int64_t s_out;
  void* conv_state;       int64_t s_cs_slot, s_cs_chan, s_cs_tok;
  const void* conv_weight; int64_t s_w_chan, s_w_tap;
  const int32_t* qsl;
  const int32_t* slots;
  const int32_t* accepted;
  const int32_t* record_rows;               // may be null
  int32_t* counter;
  int32_t B, H, Q, N, R, T, null_id;
  int32_t out_bf16, kg_bf16, w_bf16;
  int32_t use_lb;
  float lb;
  int32_t n_items;
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
  int32_t L, B, H, Q, null_id;
  int64_t N, R;
  int32_t kg_bf16;
};

// Launchers (return a hipError_t as int).  `grid` <= 0 means the default.
int launch_verify(const VerifyParams& p, int D, bool act_bf16, int grid,
                  hipStream_t stream);
int launch_commit(const CommitParams& p, int D, hipStream_t stream);
int launch_reset_counter(int32_t* counter, int n, hipStream_t stream);

}  // namespace kda
