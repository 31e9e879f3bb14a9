// Multi-layer RecoverSSM commit for gfx950: folds each request's first n
// accepted draft positions into its fp32 checkpoint, for every KDA layer, in
// one launch (kernels page `cute_recoverssm_commit`; ops page
// `_commit_kda_state_kernel`, `KDARecoverSSMCommitContext.commit`).
//
// For one (layer, request, head), with the recorded correction c_t, raw key
// k_t and raw gate of positions t < n:
//   S_n = S_0 diag(Gam) + sum_{t<n} c_t (k_hat_t * Suf_t)^T
//   Gam = prod_{t<n} d_t,   Suf_t = prod_{t<s<n} d_s,   d = exp(gate)
// which is the n-step recurrence S <- S diag(d_t) + c_t k_hat_t^T written out.
// The per-column vectors (Gam, k_hat_t * Suf_t) are built once per head in
// LDS; each state element then costs 1 + n multiply-adds, so the kernel is a
// streaming read-modify-write of the 64 KiB tile: 16-byte non-temporal
// loads issued after the small record loads, stores to the final slot.
//
// Align mode (prefix caching; ops page `_commit_kda_state_kernel` with
// ALIGN_MODE): a request may also store the state after its first m
// positions at a boundary slot,
//   S_m = S_0 diag(Gam_m) + sum_{t<m} c_t (k_hat_t * Suf^m_t)^T,
// built from the same tile in registers with a second set of column vectors
// (a separate instantiation, so the plain commit carries none of it).
//
// Schedules: by default one workgroup per (head, request, layer) on a 3-D
// grid, taken in XCD-aware order: the dispatcher hands consecutive
// workgroups to the 8 XCDs in turn, so workgroup i processes item
// (i mod 8) * n/8 + i/8 and each XCD streams one contiguous eighth of the
// items (heads fastest, then requests, then layers), keeping the heads of
// one slot and their records together in that XCD's L2 (8% faster on a
// 24-layer commit, 1.5% on one layer).  With grid > 0, a persistent grid of
// that many workgroups walks the items with a stride.
#include <type_traits>

#include "kda_step.hpp"

namespace kda {
namespace {

template <int D, int QMAX>
struct CommitCfg {
  // 1024 threads at D = 128: 4 float4 of the tile per thread and 16 waves
  // per workgroup keep the read-modify-write stream busy; with the
  // XCD-aware order this is 5% faster than 512 threads (190 vs 201 us on the
  // 256-request batch) and 256 threads (204 us).  At Q = 16 the persistent
  // loop would spill at that size: 512 threads there.
  static constexpr int NT =
      D >= 128 ? (QMAX >= 16 ? 512 : 1024) : (D == 64 ? 128 : 64);
  static constexpr int L = D / 4;           // lanes per state row (float4)
  static constexpr int RPP = NT / L;        // rows per pass
  static constexpr int PASSES = D / RPP;
  static constexpr int CW = (D + 63) / 64;  // waves holding columns
  static constexpr int CS = QMAX + 4;       // padded row of corrections
  static constexpr int JC = (QMAX * D + NT - 1) / NT;  // corrections/thread
  static_assert(RPP * PASSES == D, "tile rows");
};

template <int D, int QMAX, bool ALIGN>
struct BoundarySmem {
  float wb[QMAX][D];       // k_hat_t * Suf^m_t (0 for t >= m)
  float gamb[D];           // Gam_m
};
template <int D, int QMAX>
struct BoundarySmem<D, QMAX, false> {};

template <int D, int QMAX, bool ALIGN>
struct alignas(16) CommitSmem {
  using C = CommitCfg<D, QMAX>;
  float w[QMAX][D];        // k_hat_t * Suf_t
  float gam[D];            // Gam
  float cT[D * C::CS];     // corrections, row v: c_0..c_{Q-1}
  float red[C::CW][QMAX];  // wave partial sums of |k_t|^2
  BoundarySmem<D, QMAX, ALIGN> bd;
};

// Conv histories of one head for the fused step: channels part*H*D + h*D + d
// (part < 3: the q, k and v blocks), W - 1 entries each for the final slot
// and the boundary slot, held as 32-bit words between the loads and the
// stores.
template <int D, int NT>
struct HeadHistories {
  static constexpr int CH = (3 * D + NT - 1) / NT;  // channels per thread
  uint32_t fin[CH][kConvWidth - 1];
  uint32_t bnd[CH][kConvWidth - 1];
};

template <int D, int NT, class T>
__device__ __forceinline__ void load_head_histories(
    HeadHistories<D, NT>& hh, const T* src, int64_t s_ch, int64_t s_tok,
    int64_t head_ch, int64_t part_ch, int n, int m, bool bnd) {
#pragma unroll
  for (int c = 0; c < HeadHistories<D, NT>::CH; ++c) {
    const int j = int(threadIdx.x) + c * NT;
    if (j < 3 * D) {
      const int part = j / D;
      const T* row = src + (head_ch + part * part_ch + (j - part * D)) * s_ch;
      const ConvHistory<T> a = load_history(row, s_tok, n);
#pragma unroll
      for (int i = 0; i < kConvWidth - 1; ++i) hh.fin[c][i] = a.v[i];
      if (bnd) {
        const ConvHistory<T> e = load_history(row, s_tok, m);
#pragma unroll
        for (int i = 0; i < kConvWidth - 1; ++i) hh.bnd[c][i] = e.v[i];
      }
    }
  }
}

template <int D, int NT, class T>
__device__ __forceinline__ void store_head_histories(
    const HeadHistories<D, NT>& hh, T* fdst, T* bdst, int64_t s_ch,
    int64_t s_tok, int64_t head_ch, int64_t part_ch) {
#pragma unroll
  for (int c = 0; c < HeadHistories<D, NT>::CH; ++c) {
    const int j = int(threadIdx.x) + c * NT;
    if (j < 3 * D) {
      const int part = j / D;
      const int64_t off = (head_ch + part * part_ch + (j - part * D)) * s_ch;
      if (bdst) {                                       // boundary first
        ConvHistory<T> e;
#pragma unroll
        for (int i = 0; i < kConvWidth - 1; ++i) e.v[i] = T(hh.bnd[c][i]);
        store_history(bdst + off, s_tok, e);
      }
      ConvHistory<T> a;
#pragma unroll
      for (int i = 0; i < kConvWidth - 1; ++i) a.v[i] = T(hh.fin[c][i]);
      store_history(fdst + off, s_tok, a);
    }
  }
}

// The fused step's compaction for one (layer, request, head): `load` issues
// the reads, `store` the writes (after every read of the item).
template <int D, int NT>
struct HeadCompaction {
  HeadHistories<D, NT> hh;
  bool on = false, bnd = false;
  int64_t base = 0;
  int64_t s_slot = 0, s_ch = 0, s_tok = 0, head_ch = 0, part_ch = 0;
  int slot = 0, f = 0, bslot = 0;

  __device__ __forceinline__ void load(const CommitParams& p, int l, int h,
                                       int slot_, int n, int f_, int bslot_,
                                       int m) {
    on = p.conv_tables != nullptr;
    if (!on) return;
    const int64_t L = p.L;
    base = p.conv_tables[l];
    s_slot = p.conv_tables[L + l];
    s_ch = p.conv_tables[2 * L + l];
    s_tok = p.conv_tables[3 * L + l];
    head_ch = int64_t(h) * D;
    part_ch = int64_t(p.H) * D;
    slot = slot_;
    f = f_;
    bslot = bslot_;
    bnd = bslot_ >= 0 && m >= 1;
    if (p.conv_elem == 2)
      load_head_histories<D, NT>(
          hh, global_addr<const uint16_t>(base) + slot * s_slot, s_ch,
          s_tok, head_ch, part_ch, n, m, bnd);
    else
      load_head_histories<D, NT>(
          hh, global_addr<const uint32_t>(base) + slot * s_slot, s_ch,
          s_tok, head_ch, part_ch, n, m, bnd);
  }

  __device__ __forceinline__ void store(const CommitParams& p) {
    if (!on) return;
    if (p.conv_elem == 2) {
      uint16_t* b16 = global_addr<uint16_t>(base);
      store_head_histories<D, NT>(hh, b16 + f * s_slot,
                                  bnd ? b16 + bslot * s_slot : nullptr, s_ch,
                                  s_tok, head_ch, part_ch);
    } else {
      uint32_t* b32 = global_addr<uint32_t>(base);
      store_head_histories<D, NT>(hh, b32 + f * s_slot,
                                  bnd ? b32 + bslot * s_slot : nullptr, s_ch,
                                  s_tok, head_ch, part_ch);
    }
  }
};

template <int D, int NT>
struct NoCompaction {
  __device__ __forceinline__ void load(const CommitParams&, int, int, int,
                                       int, int, int, int) {}
  __device__ __forceinline__ void store(const CommitParams&) {}
};

// Commit of one (layer, request, head).  Returns whether it used LDS (a
// skipped item returns before touching it).  STEP: the fused commit step
// (plan inline, and the conv compaction of this head).
template <int D, int QMAX, bool ALIGN, bool STEP>
__device__ __forceinline__ bool commit_item(const CommitParams& p,
                                            CommitSmem<D, QMAX, ALIGN>& sm,
                                            int l, int b, int h) {
  using C = CommitCfg<D, QMAX>;
  const int tid = threadIdx.x;
  const int slot = p.slots[b];
  int n, f;
  // boundary slot (align mode): -1 when there is none to store
  int bslot = -1, m = 0;
  if constexpr (STEP) {
    const RequestPlan pl = plan_request(p.plan, b);
    if (l == 0 && h == 0 && tid == 0) store_plan(p.plan, b, pl);
    if (slot <= p.null_id || slot < 0 || slot >= p.N) return false;
    n = pl.n;
    if (n == 0) return false;
    f = pl.final_slot;
    if (f <= p.null_id || f < 0 || f >= p.N) return false;
    if constexpr (ALIGN) {
      bslot = pl.bnd;
      m = min(max(pl.blen, 0), n);
      if (bslot <= p.null_id || bslot < 0 || bslot >= p.N) bslot = -1;
    }
  } else {
    if (slot <= p.null_id || slot < 0 || slot >= p.N) return false;
    n = min(max(p.commit_lens[b], 0), p.Q);
    if (n == 0) return false;
    f = p.final_slots ? p.final_slots[b] : slot;
    if (f <= p.null_id || f < 0 || f >= p.N) return false;
    if constexpr (ALIGN) {
      bslot = p.bnd_slots[b];
      m = min(max(p.bnd_lens[b], 0), n);
      if (bslot <= p.null_id || bslot < 0 || bslot >= p.N) bslot = -1;
    }
  }
  const int r = p.record_rows ? p.record_rows[b] : slot;
  // The compaction's reads come next (after the record row, whose load is
  // waited for at once), so that the record loads below retire after them
  // and its writes can go out once those have landed.
  std::conditional_t<STEP, HeadCompaction<D, C::NT>, NoCompaction<D, C::NT>>
      conv;
  conv.load(p, l, h, slot, n, f, bslot, m);
  if (r < 0 || r >= p.R) {
    conv.store(p);
    return false;
  }

  float* state = global_addr<float>(p.state_base[l]);
  const int64_t sbs = p.state_bs[l];
  const float* src = state + int64_t(slot) * sbs + int64_t(h) * p.s_state_head;
  float* dst = state + int64_t(f) * sbs + int64_t(h) * p.s_state_head;
  float* bdst = state + int64_t(bslot < 0 ? f : bslot) * sbs +
                int64_t(h) * p.s_state_head;

  // Records of this head.
  const float* corr = global_addr<const float>(p.corr_base[l]) +
                      int64_t(r) * p.corr_bs[l] + int64_t(h) * p.s_c_head;
  const int64_t kg_off = int64_t(r) * p.kg_bs[l] + int64_t(h) * p.s_kg_head;
  const void* kg = global_addr<const char>(p.kg_base[l]);
  const bool kg_bf16 = p.kg_bf16 != 0;

  // Small loads first (vector-memory counters retire in issue order): the
  // corrections (transposed so that a row's values are contiguous), the raw
  // keys and gates, the gate parameters; then the state tile.
  float cv[C::JC];
#pragma unroll
  for (int jj = 0; jj < C::JC; ++jj) {
    const int j = tid + jj * C::NT;
    const int t = j / D, v = j - t * D;
    cv[jj] = (j < QMAX * D && t < n) ? corr[int64_t(t) * p.s_c_pos + v]
                                     : 0.0f;
  }

  // Per column k: raw keys and decays of the committed positions.
  const float Ah =
      __expf(p.A_log[int64_t(l) * p.s_A_l + int64_t(h) * p.s_A_h]);
  const bool use_lb = p.use_lb[l] != 0;
  const float lb = p.lb[l];
  const bool col_ok = tid < D;
  const float bias =
      col_ok ? p.dt_bias[int64_t(l) * p.s_dt_l + int64_t(h) * p.s_dt_h +
                         int64_t(tid) * p.s_dt_d]
             : 0.0f;
  float kr[QMAX], gr[QMAX], dd[QMAX];
#pragma unroll
  for (int t = 0; t < QMAX; ++t) {
    kr[t] = 0.0f;
    gr[t] = 0.0f;
    if (col_ok && t < n) {
      const int64_t o = kg_off + int64_t(t) * p.s_kg_pos;
      kr[t] = ld_elem(kg, o + tid, kg_bf16);
      gr[t] = ld_elem(kg, o + D + tid, kg_bf16);
    }
  }

  // The state tile: lane group rg owns rows rg, rg+RPP, ...
  const int lg = tid % C::L, rg = tid / C::L;
  const int col = 4 * lg;
  f4 st[C::PASSES];
#pragma unroll
  for (int pp = 0; pp < C::PASSES; ++pp)
    st[pp] = ld_stream(src + (pp * C::RPP + rg) * D + col);

#pragma unroll
  for (int jj = 0; jj < C::JC; ++jj) {
    const int j = tid + jj * C::NT;
    const int t = j / D, v = j - t * D;
    if (j < QMAX * D) sm.cT[v * C::CS + t] = cv[jj];
  }
  conv.store(p);
#pragma unroll
  for (int t = 0; t < QMAX; ++t)
    dd[t] = (col_ok && t < n)
                ? __expf(kda_gate(gr[t] + bias, Ah, use_lb, lb))
                : 1.0f;
  const int wave = tid / 64, lane = tid % 64;
  if (wave < C::CW) {
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      const float s = wave_sum(kr[t] * kr[t]);
      if (lane == 0) sm.red[wave][t] = s;
    }
  }
  lds_barrier();

  if (col_ok) {
    float suf = 1.0f, sufb = 1.0f;
#pragma unroll
    for (int t = QMAX - 1; t >= 0; --t) {
      float sk = 0.0f;
#pragma unroll
      for (int w = 0; w < C::CW; ++w) sk += sm.red[w][t];
      const float kh = kr[t] * rsqrtf(sk + kNormEps);
      sm.w[t][tid] = kh * suf;
      suf *= dd[t];
      if constexpr (ALIGN) {
        sm.bd.wb[t][tid] = t < m ? kh * sufb : 0.0f;
        if (t < m) sufb *= dd[t];
      }
    }
    sm.gam[tid] = suf;
    if constexpr (ALIGN) sm.bd.gamb[tid] = sufb;
  }
  lds_barrier();

  const f4 g4 = *reinterpret_cast<const f4*>(&sm.gam[col]);
  f4 w4[QMAX];
#pragma unroll
  for (int t = 0; t < QMAX; ++t)
    w4[t] = *reinterpret_cast<const f4*>(&sm.w[t][col]);
#pragma unroll
  for (int pp = 0; pp < C::PASSES; ++pp) {
    const int row = pp * C::RPP + rg;
    f4 acc = st[pp] * g4;
    const float* cr = &sm.cT[row * C::CS];
    if constexpr (ALIGN) {
      // the boundary state first, from the same tile
      if (bslot >= 0) {
        f4 bacc = st[pp] * *reinterpret_cast<const f4*>(&sm.bd.gamb[col]);
#pragma unroll
        for (int t = 0; t < QMAX; ++t) {
          if (t < m) {
            const float c = cr[t];
            const f4 wb = *reinterpret_cast<const f4*>(&sm.bd.wb[t][col]);
            bacc.x = fmaf(c, wb.x, bacc.x);
            bacc.y = fmaf(c, wb.y, bacc.y);
            bacc.z = fmaf(c, wb.z, bacc.z);
            bacc.w = fmaf(c, wb.w, bacc.w);
          }
        }
        st_stream(bdst + row * D + col, bacc);
      }
    }
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      if (t < n) {
        const float c = cr[t];
        acc.x = fmaf(c, w4[t].x, acc.x);
        acc.y = fmaf(c, w4[t].y, acc.y);
        acc.z = fmaf(c, w4[t].z, acc.z);
        acc.w = fmaf(c, w4[t].w, acc.w);
      }
    }
    st_stream(dst + row * D + col, acc);
  }
  return true;
}

// One workgroup per item: blockIdx = (head, request, layer).
template <int D, int QMAX, bool ALIGN, bool STEP>
__global__ void __launch_bounds__((CommitCfg<D, QMAX>::NT))
    kda_commit_grid_kernel(CommitParams p) {
  __shared__ CommitSmem<D, QMAX, ALIGN> sm;
  // XCD-aware order: consecutive workgroups go to the 8 XCDs in turn, so
  // let XCD k take the k-th eighth of the items in order.
  const int per_layer = p.B * p.H;
  const int n = p.L * per_layer;
  const int lin = int(blockIdx.x) + p.H * (int(blockIdx.y) + p.B * int(blockIdx.z));
  int item = lin;
  if ((n & 7) == 0) item = (lin & 7) * (n >> 3) + (lin >> 3);
  const int l = item / per_layer;
  const int rem = item - l * per_layer;
  const int b = rem / p.H;
  commit_item<D, QMAX, ALIGN, STEP>(p, sm, uniform(l), uniform(b),
                                    uniform(rem - b * p.H));
}

// Persistent grid: workgroup g takes items g, g + gridDim.x, ... in
// (layer, request, head) order, heads fastest.
template <int D, int QMAX, bool ALIGN, bool STEP>
__global__ void __launch_bounds__((CommitCfg<D, QMAX>::NT))
    kda_commit_strided_kernel(CommitParams p) {
  __shared__ CommitSmem<D, QMAX, ALIGN> sm;
  const int per_layer = p.B * p.H;
  const int n_items = p.L * per_layer;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int l = uniform(item / per_layer);
    const int rem = item - l * per_layer;
    const int b = uniform(rem / p.H);
    const int h = uniform(rem - b * p.H);
    // LDS is reused by the next item: wait until every thread is done.
    if (commit_item<D, QMAX, ALIGN, STEP>(p, sm, l, b, h)) lds_barrier();
  }
}

template <int D, int QMAX, bool ALIGN, bool STEP>
int launch_cqa(const CommitParams& p, hipStream_t stream) {
  using C = CommitCfg<D, QMAX>;
  const int64_t items = int64_t(p.L) * p.B * p.H;
  if (items > 0x7fffffff) return int(hipErrorInvalidValue);
  if (p.grid <= 0 && p.B <= 65535 && p.L <= 65535) {
    launch_kernel((kda_commit_grid_kernel<D, QMAX, ALIGN, STEP>),
                  dim3(p.H, p.B, p.L), dim3(C::NT), 0, stream, p);
  } else {
    const int64_t g = p.grid > 0 ? p.grid : 4096;
    launch_kernel((kda_commit_strided_kernel<D, QMAX, ALIGN, STEP>),
                  dim3(unsigned(g < items ? g : items)), dim3(C::NT), 0,
                  stream, p);
  }
  return int(hipGetLastError());
}

// Align mode when boundary slots are given (or, in the fused step, when the
// plan has a block table).
template <int D, int QMAX>
int launch_cq(const CommitParams& p, hipStream_t stream) {
  if (p.step)
    return p.plan.table ? launch_cqa<D, QMAX, true, true>(p, stream)
                        : launch_cqa<D, QMAX, false, true>(p, stream);
  return p.bnd_slots ? launch_cqa<D, QMAX, true, false>(p, stream)
                     : launch_cqa<D, QMAX, false, false>(p, stream);
}

template <int D>
int launch_cd(const CommitParams& p, hipStream_t stream) {
  if (p.Q <= 4) return launch_cq<D, 4>(p, stream);
  if (p.Q <= 8) return launch_cq<D, 8>(p, stream);
  return launch_cq<D, 16>(p, stream);
}

}  // namespace

int launch_commit(const CommitParams& p, int D, hipStream_t stream) {
  switch (D) {
    case 16: return launch_cd<16>(p, stream);
    case 32: return launch_cd<32>(p, stream);
    case 64: return launch_cd<64>(p, stream);
    case 128: return launch_cd<128>(p, stream);
    default: return int(hipErrorInvalidValue);
  }
}

}  // namespace kda
