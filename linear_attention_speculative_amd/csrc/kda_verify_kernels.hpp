// Fused short-conv update + RecoverSSM speculative verify of one KDA layer,
// for gfx950 (wave64).  One workgroup handles one (request, head) work item:
// by default one workgroup per item (hardware dispatch); optionally a
// persistent grid whose workgroups draw items from a ticket counter.
//
// What is computed (ops page `_kda_recoverssm_verify_kernel` with the conv
// update of the kernels page's `CuteRecoverSSMVerify`): for draft positions
// t < q of a request, starting from the checkpoint S (V x K, fp32),
//   S_t     = S_{t-1} diag(d_t) + c_t k_t^T      (d_t = exp(g_t), k normalised)
//   c_t     = beta_t (v_t - S_{t-1} diag(d_t) k_t)
//   o_t     = S_t q_t                              (q normalised, * K^-1/2)
// The checkpoint is never written, so the kernel never materialises S_t.
// Unrolling the recurrence gives, with Gam_t = prod_{r<=t} d_r and
// P_{s,t} = prod_{s<r<=t} d_r (no division anywhere):
//   S_{t-1} diag(d_t) k_t = S (Gam_t * k_t) + sum_{s<t} c_s <k_s, P_{s,t} k_t>
//   o_t                   = S (Gam_t * q_t) + sum_{s<=t} c_s <k_s, P_{s,t} q_t>
// so each state row needs 2Q dot products against the read-only checkpoint
// (streamed from HBM once) plus a Q x Q triangular solve per row that uses
// only per-head K-vector quantities.  That halves the per-element work of
// the step-by-step form and keeps the state tile out of the critical path.
//
// With several items resident per compute unit the HBM traffic sets the
// pace only if every per-item overhead is small, so: addresses are 32-bit
// offsets from wave-uniform 64-bit bases; sigmoid/softplus use the hardware
// exp, log and reciprocal; the K-dimension sums are reduced across lanes,
// several scalars per step; the row dot products are reduced with a
// transposing DPP reduction that leaves one finished value per lane.
//
// Phases of one item (LDS barriers between them):
//   0  issue the small loads (conv history, new inputs, taps, gate, beta),
//      then the 16-byte streaming loads of the state tile into registers
//      (vector-memory counters retire in issue order, so the small loads go
//      first and the prologue computes while the tile streams in); conv
//      update of the head's 3D channels (history at offset a-1 of the conv
//      state, SiLU), roll the conv state in place, key record; gate decays
//      and the raw-gate half of the key record; sigmoid(beta).
//   1  per column k: |k_t|^2, |q_t|^2 and the pairwise terms
//      <k_s, P_{s,t} k_t>, <k_s, P_{s,t} q_t>, summed over k.  D >= 64: each
//      wave sums over its 64 columns by a transposing lane reduction (one
//      LDS word per scalar and wave) and the unnormalised column vectors
//      Gam_t k_t, Gam_t q_t go to LDS; else an LDS tree.
//   2  the Q x Q coefficient matrices and the 2Q norm factors (below
//      D = 64 also the normalised column vectors).
//   3  dot products of every state row with the 2Q column vectors;
//      transposing reduction over the lanes that share a row; row results
//      to LDS.
//   4  one thread per row: row sums scaled by their norm factors, triangular
//      solve for c_t, outputs o_t; stores of out and of the correction record
//      (coalesced along V).
#pragma once

#include <utility>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

// DV: state rows (values) one workgroup handles, D for a whole head or a
// V-tile of D / VT rows.  The per-row arithmetic does not depend on DV (same
// lanes per row, same column order, same reduction tree), so a V-tiled
// launch gives the same bits as an untiled one.
template <int D, int QMAX, int DV = D>
struct VerifyCfg {
  static constexpr int NT_HEAD = D >= 128 ? 256 : (D == 64 ? 128 : 64);
  // lanes sharing one state row in the dot-product phase (8 at D = 128:
  // 16 columns per lane, three transposing-reduction steps instead of
  // four; 2% faster at Q = 8, the same at Q = 4)
  static constexpr int L = D >= 128 ? 8 : D >= 64 ? 16 : (D == 32 ? 8 : 4);
  // A V-tile takes one pass of L lanes per row where it can, but never
  // fewer threads than columns (the column phase has one thread per
  // column) or than one wave.
  static constexpr int NT_MIN = D > 64 ? D : 64;
  static constexpr int NT =
      DV == D ? NT_HEAD
              : (DV * L < NT_MIN ? NT_MIN
                                 : (DV * L > NT_HEAD ? NT_HEAD : DV * L));
  static constexpr int RPP = NT / L;           // rows per pass
  static constexpr int PASSES = DV / RPP;      // passes over the tile
  static constexpr int CHUNKS = D / (4 * L);   // float4 per lane per row
  static constexpr int NVAL = 2 * PASSES;      // row sums per lane, per t
  // Column phase: D >= 64 gives NG groups of D threads (whole waves), each
  // computing a share of the partial sums; below 64 one group does all.
  static constexpr int NG = D >= 64 ? NT / D : 1;
  static constexpr int NM = QMAX * (QMAX - 1) / 2;  // <k_s, P k_t>, s < t
  static constexpr int NN = QMAX * (QMAX + 1) / 2;  // <k_s, P q_t>, s <= t
  static constexpr int NV = 2 * QMAX + NM + NN;     // reduced scalars
  static constexpr int DS = 2 * QMAX + 4;           // padded row of dots
  // Column sums, D >= 64: each wave reduces its group's NS scalars over its
  // 64 columns with a transposing lane reduction (16 scalars at a time),
  // one LDS word per scalar and wave, one barrier.  Otherwise an LDS
  // reduction tree: columns summed in chunks of CH, NB scalars at a time
  // (NV / NB batches of two barriers each: eight at Q = 16, where they took
  // 28 of an item's 48 us).  The ticket loop keeps the tree at Q = 16: the
  // lane reduction's 144 scalars per group would spill its registers.
  static constexpr bool WAVE_COLS = D >= 64;
  static constexpr bool TREE = !WAVE_COLS || QMAX > 8;  // tree space needed
  static constexpr int WPG = WAVE_COLS ? D / 64 : 1;  // waves per group
  static constexpr int NS = (NV + NG - 1) / NG;       // scalars per group
  static constexpr int CH = D >= 32 ? 32 : D;
  static constexpr int NCH = D / CH;
  static constexpr int NB = NV * D <= 5120 ? NV : 5120 / D;
  static constexpr int PART =
      TREE ? (NB * D > D * DS ? NB * D : D * DS) : D * DS;
  // conv channels: q and k of the whole head, v of this workgroup's rows
  static constexpr int NCONV = 2 * D + DV;
  static constexpr int JC = (NCONV + NT - 1) / NT;  // conv channels/thread
  static constexpr int JG = (QMAX * D + NT - 1) / NT;  // gate values/thread
  // Register budget: 4 waves per SIMD up to Q = 8 (LDS allows 4
  // workgroups per CU; at Q = 8 this needs the register savings of phases
  // 1-3 below: 7% faster than 3 waves), 1 at Q = 16.  The ticket loop
  // carries more live state: 3 up to Q = 4, 2 at Q = 8.  No instantiation
  // may spill (the build checks it).
  static constexpr int MIN_WAVES = QMAX >= 16 ? 1 : 4;
  static constexpr int TICKET_MIN_WAVES = QMAX >= 16 ? 1 : QMAX >= 8 ? 2 : 3;
  static_assert(PASSES >= 1 && RPP * PASSES == DV, "tile rows");
  static_assert(NT >= D || D < 64, "one thread per column");
  static_assert(CHUNKS * 4 * L == D, "tile columns");
  static_assert(NVAL <= L, "one row sum per lane");
};

template <int D, int QMAX>
struct alignas(16) VerifySmem {
  using C = VerifyCfg<D, QMAX>;
  float y[3][QMAX][D];           // conv outputs q | k | v, positions < q
  float dec[QMAX][D];            // decays d_t
  // Gam_t k_hat_t, then Gam_t q_hat_t: written in phase 2 over y's q and k
  // rows, which phase 1 has read into registers (only v is read later)
  __device__ float (*vec())[D] {
    return reinterpret_cast<float (*)[D]>(&y[0][0][0]);
  }
  // column partial sums [NB][D] (phase 1, D < 64), then per row:
  // S.(Gam k_hat_t), S.(Gam q_hat_t) [D][DS] (phases 3-4)
  alignas(16) float part[C::PART];  // (read as float4)
  // column sums: per wave and scalar of its group (D >= 64), else chunk
  // sums of the column partials
  float red[C::WAVE_COLS && (C::NT_HEAD / 64) * C::NV > C::NV * C::NCH
                ? (C::NT_HEAD / 64) * C::NV
                : C::NV * C::NCH];
  float Mc[QMAX][QMAX];          // <k_hat_s, P_{s,t} k_hat_t>, s < t
  float Nc[QMAX][QMAX];          // <k_hat_s, P_{s,t} q_hat_t>, s <= t
  // column sums by lane reduction: the unnormalised column vectors
  // Gam_t k_t, Gam_t q_t (written in phase 1) and the norm factors that
  // phase 4 applies to the row sums
  alignas(16) float uvec[C::WAVE_COLS ? 2 * QMAX : 1][D];  // (float4)
  float nrm[2][QMAX];
  float beta[QMAX];
  int ticket[2];
};

// LDS of the deferred flush (fused commit of the previous step's pending
// positions before the verify): per column the decay product Gam and the
// vectors k_hat_t * Suf_t, per row the pending corrections.
template <int D, int QMAX, bool FLUSH>
struct alignas(16) FlushSmem {
  float gam[D];               // Gam = prod_{t<n} d_t
  float w[QMAX][D];           // raw keys, then k_hat_t * Suf_t
  float dec[QMAX][D];         // pending decays d_t
  float cT[D][QMAX + 1];      // corrections, row v: c_0 .. c_{n-1}
  float ksum[QMAX];           // |k_t|^2
};
template <int D, int QMAX>
struct FlushSmem<D, QMAX, false> {};

// Index of the pair terms in the reduction vector.
template <int QMAX>
__device__ __forceinline__ constexpr int idx_m(int t, int s) {
  return 2 * QMAX + t * (t - 1) / 2 + s;
}
template <int QMAX>
__device__ __forceinline__ constexpr int idx_n(int t, int s) {
  return 2 * QMAX + QMAX * (QMAX - 1) / 2 + t * (t + 1) / 2 + s;
}

// The verify's output, correction and record stores: plain, or streamed
// past the caches (non-temporal) at Q >= 8, where that measured 3% faster on
// the 24-layer batch (at Q = 4 it measured 1% slower).
template <int QMAX, class T>
__device__ __forceinline__ void put_result(T* p, T v) {
  if constexpr (QMAX >= 8)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// Wave-uniform description of one (request, head) work item.
struct Item {
  int b, h, bos, q, slot, r, a;
  int v0;        // first state row (value) of a V-tile, else 0
  bool valid, live, rec_ok;
  bool slot_ok;  // the slot is live, whatever the window length
};

// The item past the end of a schedule: no view of it holds any byte.
__device__ __forceinline__ Item no_item() {
  Item it{};
  it.v0 = 0;
  it.valid = false;
  it.live = false;
  it.rec_ok = false;
  it.slot_ok = false;
  return it;
}

__device__ __forceinline__ Item load_item(const VerifyParams& p, int b,
                                          int h) {
  Item it;
  it.valid = true;
  it.b = b;
  it.h = h;
  it.v0 = 0;
  int bos, eos, slot, acc;
  sload4(p.qsl + b, p.qsl + b + 1, p.slots + b, p.accepted + b, bos, eos,
         slot, acc);
  // Token rows outside [0, T) are never touched (memory-safety clamp).
  it.bos = bos;
  it.q = (bos < 0 || bos >= p.T) ? 0
                                 : min(min(max(eos - bos, 0), p.Q), p.T - bos);
  it.slot = slot;
  it.slot_ok = slot > p.null_id && slot >= 0 && slot < p.N;
  it.live = it.q > 0 && it.slot_ok;
  it.a = min(max(acc, 1), p.Q);
  it.r = p.record_rows ? sload1(p.record_rows + b) : slot;
  it.rec_ok = it.r >= 0 && it.r < p.R;
  return it;
}

// Conv channel covered by slot j < NCONV of a workgroup: the head's q and k
// channels first (j < 2D), then the value channels of its rows [v0, v0+DV).
template <int D, int DV>
__device__ __forceinline__ void conv_slot(int j, int v0, int& part, int& d) {
  part = j / D;
  d = j - part * D;
  if constexpr (DV != D) d += part == 2 ? v0 : 0;
}

// Per-head constants, raw: conv taps of the workgroup's channels (f32 bits,
// or a bf16 in the low half), dt_bias, A_log.
template <int D, int QMAX, int DV = D>
struct HeadRegs {
  using C = VerifyCfg<D, QMAX, DV>;
  uint32_t w[C::JC][4];
  float gb[C::JG];
  float alog;
};

// Raw registers of one item's small loads: conv history, new inputs, gate
// inputs, beta.  Conversions happen where the values are used, so that no
// instruction waits for these loads where they are issued.
template <int D, int QMAX, bool ACT_BF16, int DV = D>
struct Small {
  using C = VerifyCfg<D, QMAX, DV>;
  using AT = typename Act<ACT_BF16>::T;
  // dwords of one channel's conv-state row (QMAX + 2 elements)
  static constexpr int RD = (QMAX + 2) * int(sizeof(AT)) / 4;
  AT hist[C::JC][3];        // history, element by element
  uint32_t row[C::JC][RD];  // or the whole row (contiguous-row layout)
  AT xs[C::JC][QMAX];
  AT gv[C::JG];
  AT bv;
};

// The state tile of one item in registers: lane lg of row group rg holds
// rows v0 + pp * RPP + rg, columns c * 4L + 4 lg .. + 3.
template <int D, int QMAX, int DV = D>
using Tile =
    f4[VerifyCfg<D, QMAX, DV>::PASSES][VerifyCfg<D, QMAX, DV>::CHUNKS];

template <int D, int QMAX, int DV = D>
__device__ __forceinline__ void load_head(const VerifyParams& p, int h,
                                          HeadRegs<D, QMAX, DV>& hr,
                                          int v0 = 0) {
  using C = VerifyCfg<D, QMAX, DV>;
  const int tid = fresh_tid();
  const int HD = p.H * D;
  const bool w_bf16 = (p.flags & kWBf16) != 0;
  const bool conv = (p.flags & kNoConv) == 0;
#pragma unroll
  for (int jj = 0; jj < C::JC; ++jj) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hr.w[jj][i] = 0;
    const int j = tid + jj * C::NT;
    if (conv && j < C::NCONV) {
      int part, d;
      conv_slot<D, DV>(j, v0, part, d);
      const uint32_t ch = part * HD + h * D + d;
      if (p.flags & kWRow) {
        // the channel's taps in one load; bf16 taps stay packed two per
        // word until they are used
        if (w_bf16) {
          const uint2 v = at(static_cast<const uint2*>(p.conv_weight), ch);
          hr.w[jj][0] = v.x;
          hr.w[jj][1] = v.y;
        } else {
          const uint4 v = at(static_cast<const uint4*>(p.conv_weight), ch);
          hr.w[jj][0] = v.x;
          hr.w[jj][1] = v.y;
          hr.w[jj][2] = v.z;
          hr.w[jj][3] = v.w;
        }
      } else {
        const uint32_t wo = ch * p.s_w_chan;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t o = wo + i * p.s_w_tap;
          hr.w[jj][i] =
              w_bf16 ? uint32_t(at(static_cast<const uint16_t*>(p.conv_weight), o))
                     : at(static_cast<const uint32_t*>(p.conv_weight), o);
        }
      }
    }
  }
#pragma unroll
  for (int jj = 0; jj < C::JG; ++jj)
    hr.gb[jj] = at(p.dt_bias + h * D, uint32_t((tid + jj * C::NT) % D));
  hr.alog = __int_as_float(sload1(reinterpret_cast<const int32_t*>(p.A_log) + h));
}

// Element E of a conv-state row held as dwords.
template <class AT, int E, int RD>
__device__ __forceinline__ AT row_elem(const uint32_t (&rw)[RD]) {
  if constexpr (sizeof(AT) == 2)
    return AT((rw[E / 2] >> (16 * (E % 2))) & 0xffffu);
  else
    return __uint_as_float(rw[E]);
}

// Element o + I of the row for a wave-uniform o in [0, QMAX - 1].
template <class AT, int I, int QMAX, int RD>
__device__ __forceinline__ AT row_at(const uint32_t (&rw)[RD], int o) {
  AT v = row_elem<AT, I>(rw);
  [&]<int... K>(std::integer_sequence<int, K...>) {
    ((v = (o == K + 1) ? row_elem<AT, I + K + 1>(rw) : v), ...);
  }(std::make_integer_sequence<int, QMAX - 1>{});
  return v;
}

template <class AT>
__device__ __forceinline__ uint32_t bits_of(AT v) {
  if constexpr (sizeof(AT) == 2)
    return uint32_t(v);
  else
    return __float_as_uint(v);
}

// The three history entries (positions a-1 .. a+1 of the conv state) of
// conv slot jj, as loaded.
template <int D, int QMAX, bool ACT_BF16, int DV>
__device__ __forceinline__ void history3(
    const VerifyParams& p, const Item& it,
    const Small<D, QMAX, ACT_BF16, DV>& s, int jj,
    typename Act<ACT_BF16>::T (&hv)[3]) {
  using AT = typename Act<ACT_BF16>::T;
  // each path reads only the registers its loads filled (the other set is
  // never written for this item)
  if (p.flags & kConvRow) {
    hv[0] = row_at<AT, 0, QMAX>(s.row[jj], it.a - 1);
    hv[1] = row_at<AT, 1, QMAX>(s.row[jj], it.a - 1);
    hv[2] = row_at<AT, 2, QMAX>(s.row[jj], it.a - 1);
  } else {
    hv[0] = s.hist[jj][0];
    hv[1] = s.hist[jj][1];
    hv[2] = s.hist[jj][2];
  }
}

// Roll of conv channel `ch` (conv slot jj) in place: the two newest history
// entries, then the q new inputs, at the front; positions past 2 + q keep
// their bytes.  h1, h2: history entries a and a+1.
template <int D, int QMAX, bool ACT_BF16, bool FULL, int DV>
__device__ __forceinline__ void roll_channel(
    const VerifyParams& p, const Item& it,
    const Small<D, QMAX, ACT_BF16, DV>& s, int jj, int ch,
    typename Act<ACT_BF16>::T h1, typename Act<ACT_BF16>::T h2) {
  using AT = typename Act<ACT_BF16>::T;
  using S = Small<D, QMAX, ACT_BF16, DV>;
  const int q = FULL ? QMAX : it.q;
  AT* __restrict__ cs =
      static_cast<AT*>(p.conv_state) + int64_t(it.slot) * p.s_cs_slot;
  AT* csc = cs + ch * p.s_cs_chan;
  if (p.flags & kConvRow) {
    // the whole row in one pass; its tail is written back unchanged
    constexpr int RE = QMAX + 2;
    constexpr int EW = 4 / int(sizeof(AT));  // elements per dword
    uint32_t nw[S::RD];
#pragma unroll
    for (int i = 0; i < S::RD; ++i) nw[i] = 0;
    [&]<int... E>(std::integer_sequence<int, E...>) {
      auto put = [&](auto ec) {
        constexpr int e = decltype(ec)::value;
        AT v;
        if constexpr (e == 0)
          v = h1;
        else if constexpr (e == 1)
          v = h2;
        else
          v = (e - 2 < q) ? s.xs[jj][e - 2] : row_elem<AT, e>(s.row[jj]);
        nw[e / EW] |= bits_of(v) << (32 / EW * (e % EW));
      };
      (put(std::integral_constant<int, E>{}), ...);
    }(std::make_integer_sequence<int, RE>{});
    uint32_t* wp = reinterpret_cast<uint32_t*>(csc);
#pragma unroll
    for (int i = 0; i < S::RD; ++i) wp[i] = nw[i];
  } else {
    const int s_ct = p.s_cs_tok;
    csc[0] = h1;
    csc[s_ct] = h2;
#pragma unroll
    for (int t = 0; t < QMAX; ++t)
      if (t < q) csc[(2 + t) * s_ct] = s.xs[jj][t];
  }
}

// The deferred roll of the head's q and k channels (conv slots j < 2D) by
// the last V-tile of an item to have read their history.
template <int D, int QMAX, bool ACT_BF16, bool FULL, int DV>
__device__ __forceinline__ void roll_qk(const VerifyParams& p, const Item& it,
                                        const Small<D, QMAX, ACT_BF16, DV>& s) {
  using C = VerifyCfg<D, QMAX, DV>;
  using AT = typename Act<ACT_BF16>::T;
  const int tid = fresh_tid();
  const int HD = p.H * D;
#pragma unroll
  for (int jj = 0; jj < C::JC; ++jj) {
    const int j = tid + jj * C::NT;
    if (j < 2 * D) {
      const int part = j / D, d = j - part * D;
      AT hv[3];
      history3<D, QMAX, ACT_BF16, DV>(p, it, s, jj, hv);
      roll_channel<D, QMAX, ACT_BF16, FULL, DV>(p, it, s, jj,
                                                part * HD + it.h * D + d,
                                                hv[1], hv[2]);
    }
  }
}

// Phase 0 of a live item: conv + SiLU of the workgroup's channels (the
// head's 3D, or q, k and a V-tile's values), key record, conv roll;
// `mid()` runs between the conv and the gate (the one-workgroup-per-item
// kernel issues the second half of its tile there); gate decays, raw-gate
// record half, sigmoid(beta).
// FULL: the request verifies all QMAX positions (q == QMAX), so every
// position guard folds away at compile time.  ROLL_QK false (V-tiles): the
// q and k channels, whose history every V-tile of the item reads, are not
// rolled here (roll_qk does it once all have read it), and each V-tile
// writes only its own columns of the key/gate record.
template <int D, int QMAX, bool ACT_BF16, bool FULL, int DV = D,
          bool ROLL_QK = true, class Mid>
__device__ __forceinline__ void item_front(
    const VerifyParams& p, VerifySmem<D, QMAX>& sm, const Item& it,
    const Small<D, QMAX, ACT_BF16, DV>& s, const HeadRegs<D, QMAX, DV>& hr,
    Mid&& mid) {
  using C = VerifyCfg<D, QMAX, DV>;
  using A = Act<ACT_BF16>;
  using AT = typename A::T;
  const int tid = fresh_tid();
  const int h = it.h;
  const int q = FULL ? QMAX : it.q;
  const bool rec_ok = it.rec_ok;
  const int HD = p.H * D;
  const int v0 = DV == D ? 0 : it.v0;
  const int64_t kg_off =
      int64_t(it.r) * p.s_kg_row + int64_t(h) * p.s_kg_head;
  float* __restrict__ kg32 = static_cast<float*>(p.key_gate) + kg_off;
  uint16_t* __restrict__ kg16 = static_cast<uint16_t*>(p.key_gate) + kg_off;
  const int s_kp = p.s_kg_pos;
  const bool kg_bf16 = (p.flags & kKgBf16) != 0;
  const bool w_bf16 = (p.flags & kWBf16) != 0;
  const bool conv = (p.flags & kNoConv) == 0;
  // the columns of the key/gate record this workgroup writes
  auto own_col = [&](int d) { return DV == D || (d >= v0 && d < v0 + DV); };

#pragma unroll
  for (int jj = 0; jj < C::JC; ++jj) {
    const int j = tid + jj * C::NT;
    if (j < C::NCONV) {
      int part, d;
      conv_slot<D, DV>(j, v0, part, d);
      const int ch = part * HD + h * D + d;
      float w[4];
      if (w_bf16 && (p.flags & kWRow)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          w[2 * i] = __uint_as_float(hr.w[jj][i] << 16);
          w[2 * i + 1] = __uint_as_float(hr.w[jj][i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = __uint_as_float(w_bf16 ? hr.w[jj][i] << 16 : hr.w[jj][i]);
      }
      // history: positions a-1 .. a+1 of the conv state
      AT hv[3];
      history3<D, QMAX, ACT_BF16, DV>(p, it, s, jj, hv);
      float s0 = A::f(hv[0]), s1 = A::f(hv[1]), s2 = A::f(hv[2]);
#pragma unroll
      for (int t = 0; t < QMAX; ++t) {
        if (t < q) {
          const float s3 = A::f(s.xs[jj][t]);
          float acc = w[0] * s0;
          acc = fmaf(w[1], s1, acc);
          acc = fmaf(w[2], s2, acc);
          acc = fmaf(w[3], s3, acc);
          // (the unfused entry receives the convolved value itself)
          const float yv = conv ? acc * sigmoidf_(acc) : s3;
          sm.y[part][t][d] = yv;
          if (part == 1 && rec_ok && own_col(d)) {
            if (kg_bf16)
              put_result<QMAX>(&kg16[t * s_kp + d], f32_to_bf16(yv));
            else
              put_result<QMAX>(&kg32[t * s_kp + d], yv);
          }
          s0 = s1;
          s1 = s2;
          s2 = s3;
        }
      }
      if (conv && (ROLL_QK || part == 2))
        roll_channel<D, QMAX, ACT_BF16, FULL, DV>(p, it, s, jj, ch, hv[1],
                                                  hv[2]);
    }
  }

  mid();

  const bool use_lb = (p.flags & kLowerBound) != 0;
  const float Ah = __expf(hr.alog);
#pragma unroll
  for (int jj = 0; jj < C::JG; ++jj) {
    const int j = tid + jj * C::NT;
    const int t = j / D, k = j - t * D;
    if (t < q) {
      const float g0 = A::f(s.gv[jj]);
      sm.dec[t][k] = __expf(kda_gate(g0 + hr.gb[jj], Ah, use_lb, p.lb));
      if (rec_ok && own_col(k)) {
        if (kg_bf16)
          put_result<QMAX>(&kg16[t * s_kp + D + k], f32_to_bf16(g0));
        else
          put_result<QMAX>(&kg32[t * s_kp + D + k], g0);
      }
    }
  }
  if (tid < q) sm.beta[tid] = sigmoidf_(A::f(s.bv));
}

// ---- column sums by lane reduction (D >= 64) ---------------------------------
// Scalar IDX of the reduction vector for this thread's column: |k_t|^2,
// |q_t|^2, then <k_s, P_{s,t} k_t> (s < t) and <k_s, P_{s,t} q_t> (s <= t),
// P_{s,t} = d_{s+1} ... d_t multiplied up from s + 1; IDX >= NV is 0.
template <int QMAX, int IDX>
__device__ __forceinline__ float column_scalar(const float (&kk)[QMAX],
                                              const float (&qq)[QMAX],
                                              const float (&dd)[QMAX]) {
  constexpr int NM = QMAX * (QMAX - 1) / 2;
  constexpr int NV = 2 * QMAX + NM + QMAX * (QMAX + 1) / 2;
  if constexpr (IDX >= NV) {
    return 0.0f;
  } else if constexpr (IDX < QMAX) {
    return kk[IDX] * kk[IDX];
  } else if constexpr (IDX < 2 * QMAX) {
    return qq[IDX - QMAX] * qq[IDX - QMAX];
  } else {
    constexpr bool M = IDX < 2 * QMAX + NM;
    constexpr int R = M ? IDX - 2 * QMAX : IDX - 2 * QMAX - NM;
    // R = t (t - 1) / 2 + s (M) or t (t + 1) / 2 + s
    constexpr int T = [] {
      int t = 0;
      while ((M ? (t + 1) * t / 2 : (t + 1) * (t + 2) / 2) <= R) ++t;
      return t;
    }();
    constexpr int S = R - (M ? T * (T - 1) / 2 : T * (T + 1) / 2);
    float P = 1.0f;
#pragma unroll
    for (int r = S + 1; r <= T; ++r) P *= dd[r];
    return M ? kk[S] * P * kk[T] : kk[S] * P * qq[T];
  }
}

// One 16-scalar chunk of group G (scalars G, G + NG, G + 2 NG, ...):
// transposing reduction over each 16-lane row, then across the rows, and
// lane j < 16 stores the wave's sum of the chunk's scalar j.
template <int QMAX, int G, int NG, int NS, int K, size_t... I>
__device__ __forceinline__ void column_chunk(const float (&kk)[QMAX],
                                             const float (&qq)[QMAX],
                                             const float (&dd)[QMAX],
                                             float* dst, int lane,
                                             std::index_sequence<I...>) {
  float v[16] = {column_scalar<QMAX, G + (K * 16 + int(I)) * NG>(kk, qq,
                                                                  dd)...};
  float r = transpose_sum<16, 16>(v, lane);
  r += __int_as_float(
      __builtin_amdgcn_ds_swizzle(__float_as_int(r), 0x401F));  // xor 16
  r += __int_as_float(
      __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(r)));
  const int pos = K * 16 + (lane & 15);
  if (lane < 16 && pos < NS) dst[pos] = r;
}

template <int QMAX, int G, int NG, int NS, size_t... K>
__device__ __forceinline__ void column_group(const float (&kk)[QMAX],
                                             const float (&qq)[QMAX],
                                             const float (&dd)[QMAX],
                                             float* dst, int lane,
                                             std::index_sequence<K...>) {
  (column_chunk<QMAX, G, NG, NS, int(K)>(kk, qq, dd, dst, lane,
                                         std::make_index_sequence<16>{}),
   ...);
}

// Phases 1-4 of a live item (after the barrier that publishes phase 0),
// with its state tile (rows v0 .. v0 + DV) in registers.
// PERSISTENT: the ticket loop (keeps the LDS tree at Q = 16).
template <int D, int QMAX, bool FULL, int DV = D, bool PERSISTENT = false,
          class PreDots>
__device__ __forceinline__ void item_back(const VerifyParams& p,
                                          VerifySmem<D, QMAX>& sm,
                                          const Item& it,
                                          Tile<D, QMAX, DV>& st,
                                          PreDots&& pre_dots) {
  using C = VerifyCfg<D, QMAX, DV>;
  // column sums by lane reduction (else the LDS tree)
  constexpr bool LANES = C::WAVE_COLS && (QMAX <= 8 || !PERSISTENT);
  const int tid = fresh_tid();
  const int h = it.h;
  const int q = FULL ? QMAX : it.q;
  const bool rec_ok = it.rec_ok;
  const int lg = tid % C::L;      // lane within its row group
  const int rg = tid / C::L;      // row group

  // ---- phase 1: per-column partial sums, summed over the columns ------------
  const int col = tid % D;
  const int grp = C::NG > 1 ? tid / D : 0;          // column group
  const bool col_ok = tid < D || C::NG > 1;
  float kk[QMAX], qq[QMAX], dd[QMAX];
#pragma unroll
  for (int t = 0; t < QMAX; ++t) {
    const bool ok = col_ok && t < q;
    kk[t] = ok ? sm.y[1][t][col] : 0.0f;
    qq[t] = ok ? sm.y[0][t][col] : 0.0f;
    dd[t] = ok ? sm.dec[t][col] : 1.0f;
  }
  if constexpr (LANES) {
    // wave w sums the scalars of group w / WPG over its 64 columns
    const int lane = tid & 63;
    float* dst = &sm.red[(tid >> 6) * C::NS];
    constexpr int NK = (C::NS + 15) / 16;
    // The column vectors need no norm: the dot products take Gam_t k_t and
    // Gam_t q_t, and phase 4 scales each row sum by the norm factor of its
    // position, so phase 3 starts one barrier earlier.  (Written before the
    // reduction, which then holds only its own values.)
    if (tid < D) {
      float gam = 1.0f;
#pragma unroll
      for (int t = 0; t < QMAX; ++t) {
        gam *= dd[t];
        sm.uvec[t][tid] = gam * kk[t];
        sm.uvec[QMAX + t][tid] = gam * qq[t];
      }
    }
    if (C::NG == 1 || grp == 0)
      column_group<QMAX, 0, C::NG, C::NS>(kk, qq, dd, dst, lane,
                                          std::make_index_sequence<NK>{});
    else
      column_group<QMAX, 1, C::NG, C::NS>(kk, qq, dd, dst, lane,
                                          std::make_index_sequence<NK>{});
    lds_barrier();
  } else {
#pragma unroll
    for (int v0 = 0; v0 < C::NV; v0 += C::NB) {
      // With several batches, each batch recomputes its products: opaque
      // copies of the inputs keep the compiler from carrying shared partial
      // products across the barrier in extra registers.
      if constexpr (C::NV > C::NB) {
#pragma unroll
        for (int t = 0; t < QMAX; ++t)
          asm volatile("" : "+v"(kk[t]), "+v"(qq[t]), "+v"(dd[t]));
      }
      // this thread's share of scalars [v0, v0 + NB)
      auto put = [&](int idx, float val) {
        if (idx >= v0 && idx < v0 + C::NB && idx % C::NG == grp && col_ok)
          sm.part[(idx - v0) * D + col] = val;
      };
#pragma unroll
      for (int t = 0; t < QMAX; ++t) {
        put(t, kk[t] * kk[t]);
        put(QMAX + t, qq[t] * qq[t]);
      }
#pragma unroll
      for (int s = 0; s < QMAX; ++s) {
        float P = 1.0f;
#pragma unroll
        for (int t = s; t < QMAX; ++t) {
          if (t > s) {
            P *= dd[t];
            put(idx_m<QMAX>(t, s), kk[s] * P * kk[t]);
          }
          put(idx_n<QMAX>(t, s), kk[s] * P * qq[t]);
        }
      }
      lds_barrier();
      // chunk sums: scalar v, columns [c*CH, (c+1)*CH)
      for (int task = tid; task < C::NB * C::NCH; task += C::NT) {
        const int v = task / C::NCH, c = task - v * C::NCH;
        if (v0 + v < C::NV) {
          const f4* src =
              reinterpret_cast<const f4*>(&sm.part[v * D + c * C::CH]);
          f4 acc = src[0];
#pragma unroll
          for (int i = 1; i < C::CH / 4; ++i) acc += src[i];
          sm.red[(v0 + v) * C::NCH + c] = (acc.x + acc.y) + (acc.z + acc.w);
        }
      }
      lds_barrier();
    }
  }

  // ---- phase 2: norms, column vectors, coefficient matrices ------------------
  auto total = [&](int idx) {
    float s = 0.0f;
    if constexpr (LANES) {
      const int g = idx % C::NG, pos = idx / C::NG;
#pragma unroll
      for (int w = 0; w < C::WPG; ++w)
        s += sm.red[(g * C::WPG + w) * C::NS + pos];
    } else {
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) s += sm.red[idx * C::NCH + c];
    }
    return s;
  };
  const float inv_sqrt_d = 1.0f / sqrtf(float(D));
  if constexpr (LANES) {
    // coefficient matrices and norm factors, published to phase 4 by the
    // barrier after phase 3
    for (int j = tid; j < QMAX * QMAX + QMAX; j += C::NT) {
      if (j < QMAX * QMAX) {
        const int t = j / QMAX, s = j - t * QMAX;
        const float rks = rsqrtf(total(s) + kNormEps);
        const float rkt = rsqrtf(total(t) + kNormEps);
        const float rqt = rsqrtf(total(QMAX + t) + kNormEps) * inv_sqrt_d;
        sm.Mc[t][s] = s < t ? total(idx_m<QMAX>(t, s)) * rks * rkt : 0.0f;
        sm.Nc[t][s] = s <= t ? total(idx_n<QMAX>(t, s)) * rks * rqt : 0.0f;
      } else {
        const int t = j - QMAX * QMAX;
        sm.nrm[0][t] = rsqrtf(total(t) + kNormEps);
        sm.nrm[1][t] = rsqrtf(total(QMAX + t) + kNormEps) * inv_sqrt_d;
      }
    }
    // keep phase 3's loads from being scheduled into this (registers)
    __builtin_amdgcn_sched_barrier(0);
  } else if (tid < D) {
    // q, k and the decays are read again here (thread tid's own column),
    // so that they need not stay in registers across phase 1's barriers
    float gam = 1.0f;
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      const bool ok = t < q;
      const float kt = ok ? sm.y[1][t][tid] : 0.0f;
      const float qt = ok ? sm.y[0][t][tid] : 0.0f;
      gam *= ok ? sm.dec[t][tid] : 1.0f;
      const float rk = rsqrtf(total(t) + kNormEps);
      const float rq = rsqrtf(total(QMAX + t) + kNormEps) * inv_sqrt_d;
      sm.vec()[t][tid] = gam * kt * rk;
      sm.vec()[QMAX + t][tid] = gam * qt * rq;
    }
  }
  if constexpr (!LANES) {
    for (int j = tid; j < QMAX * QMAX; j += C::NT) {
      const int t = j / QMAX, s = j - t * QMAX;
      const float rks = rsqrtf(total(s) + kNormEps);
      const float rkt = rsqrtf(total(t) + kNormEps);
      const float rqt = rsqrtf(total(QMAX + t) + kNormEps) * inv_sqrt_d;
      sm.Mc[t][s] = s < t ? total(idx_m<QMAX>(t, s)) * rks * rkt : 0.0f;
      sm.Nc[t][s] = s <= t ? total(idx_n<QMAX>(t, s)) * rks * rqt : 0.0f;
    }
    lds_barrier();
  }

  // (the deferred flush folds the pending positions into the tile here)
  pre_dots(st);

  // ---- phase 3: 2q dot products per state row ---------------------------------
  // Position-outer order: each position's two column vectors are read from
  // LDS once and applied to every pass of the register-resident tile; the
  // 2*PASSES partial sums of a lane are then reduced over its row group so
  // that lane lg ends with row sum number lg >> (log2 L - log2 NVAL).
  constexpr int SHIFT = (C::L == 16 ? 4 : C::L == 8 ? 3 : 2) -
                        (C::NVAL == 16 ? 4 : C::NVAL == 8 ? 3
                                         : C::NVAL == 4 ? 2
                                         : C::NVAL == 2 ? 1 : 0);
  const int vid = lg >> SHIFT;
  float* dslot = &sm.part[((vid >> 1) * C::RPP + rg) * C::DS +
                          (vid & 1) * QMAX];
  // (kept rolled: one position's vectors live at a time)
#pragma unroll 1
  for (int t = 0; t < q; ++t) {
    {
      // the key column, then the query column: one of them in registers at
      // a time
      float acc[C::NVAL];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        f4 va[C::CHUNKS];
#pragma unroll
        for (int c = 0; c < C::CHUNKS; ++c)
          va[c] = *reinterpret_cast<const f4*>(
              LANES ? &sm.uvec[w * QMAX + t][c * 4 * C::L + 4 * lg]
                           : &sm.vec()[w * QMAX + t][c * 4 * C::L + 4 * lg]);
#pragma unroll
        for (int pp = 0; pp < C::PASSES; ++pp) {
          float sa = 0.0f;
#pragma unroll
          for (int c = 0; c < C::CHUNKS; ++c) {
            const f4 s4 = st[pp][c];
            sa = fmaf(s4.x, va[c].x, sa);
            sa = fmaf(s4.y, va[c].y, sa);
            sa = fmaf(s4.z, va[c].z, sa);
            sa = fmaf(s4.w, va[c].w, sa);
          }
          acc[2 * pp + w] = sa;
        }
      }
      dslot[t] = transpose_sum<C::L, C::NVAL>(acc, lg);
    }
  }
  lds_barrier();

  // ---- phase 4: per-row triangular solve, outputs and corrections -------------
  if (tid < DV) {
    const int v = (DV == D ? 0 : it.v0) + tid;   // state row (value)
    // wave-uniform bases, 32-bit per-lane offsets
    float* __restrict__ corr = p.correction + int64_t(it.r) * p.s_c_row +
                               int64_t(h) * p.s_c_head;
    const int64_t ob = int64_t(it.bos) * p.s_out + h * D;
    float* __restrict__ out32 = static_cast<float*>(p.out) + ob;
    uint16_t* __restrict__ out16 = static_cast<uint16_t*>(p.out) + ob;
    const int s_cp = p.s_c_pos, s_out = p.s_out;
    const float* drow = &sm.part[tid * C::DS];
    float cc[QMAX];
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      if (t < q) {
        float u = LANES ? drow[t] * sm.nrm[0][t] : drow[t];
#pragma unroll
        for (int s = 0; s < t; ++s) u = fmaf(sm.Mc[t][s], cc[s], u);
        cc[t] = sm.beta[t] * (sm.y[2][t][v] - u);
        float o = LANES ? drow[QMAX + t] * sm.nrm[1][t]
                               : drow[QMAX + t];
#pragma unroll
        for (int s = 0; s <= t; ++s) o = fmaf(sm.Nc[t][s], cc[s], o);
        if (p.flags & kOutBf16)
          put_result<QMAX>(&at(out16, uint32_t(t * s_out + v)),
                           f32_to_bf16(o));
        else
          put_result<QMAX>(&at(out32, uint32_t(t * s_out + v)), o);
        if (rec_ok) put_result<QMAX>(&at(corr, uint32_t(t * s_cp + v)), cc[t]);
      }
    }
  }
}

// ---- deferred flush ----------------------------------------------------------
// The previous step's records of this item's record row hold n pending
// positions; the fused kernel folds them into the checkpoint (ops page
// `_commit_kda_state_kernel`, applied in place) before verifying, so the
// state tile is read once and written once for commit and verify together
// (state page, deferred commit).

// Raw pending record values: position t = j / D, element j % D.
template <int D, int QMAX>
struct PendingRegs {
  using C = VerifyCfg<D, QMAX>;
  float cv[C::JG];     // correction c_t[v]
  uint32_t kr[C::JG];  // raw key k_t[k] (f32 bits, or a bf16 in the low half)
  uint32_t gr[C::JG];  // raw gate
};

template <int D, int QMAX>
__device__ __forceinline__ void load_pending(const VerifyParams& p,
                                             const Item& it, int n,
                                             PendingRegs<D, QMAX>& pr) {
  using C = VerifyCfg<D, QMAX>;
  const int tid = fresh_tid();
  const bool kg_bf16 = (p.flags & kKgBf16) != 0;
  const float* corr = p.correction + int64_t(it.r) * p.s_c_row +
                      int64_t(it.h) * p.s_c_head;
  const int64_t kg_off =
      int64_t(it.r) * p.s_kg_row + int64_t(it.h) * p.s_kg_head;
#pragma unroll
  for (int jj = 0; jj < C::JG; ++jj) {
    const int j = tid + jj * C::NT;
    const int t = j / D, k = j % D;
    pr.cv[jj] = 0.0f;
    pr.kr[jj] = 0;
    pr.gr[jj] = 0;
    if (t < n) {
      pr.cv[jj] = corr[t * p.s_c_pos + k];
      const int64_t o = kg_off + int64_t(t) * p.s_kg_pos + k;
      if (kg_bf16) {
        pr.kr[jj] = static_cast<const uint16_t*>(p.key_gate)[o];
        pr.gr[jj] = static_cast<const uint16_t*>(p.key_gate)[o + D];
      } else {
        pr.kr[jj] = static_cast<const uint32_t*>(p.key_gate)[o];
        pr.gr[jj] = static_cast<const uint32_t*>(p.key_gate)[o + D];
      }
    }
  }
}

// Per column: Gam = prod_{t<n} d_t and w_t = k_hat_t * prod_{t<s<n} d_s;
// per row: the corrections.  Ends with a barrier.
template <int D, int QMAX>
__device__ __forceinline__ void flush_prepare(const VerifyParams& p,
                                              FlushSmem<D, QMAX, true>& fs,
                                              int n,
                                              const PendingRegs<D, QMAX>& pr,
                                              const HeadRegs<D, QMAX>& hr) {
  using C = VerifyCfg<D, QMAX>;
  const int tid = fresh_tid();
  const int lane = tid % 64, wave = tid / 64;
  const bool kg_bf16 = (p.flags & kKgBf16) != 0;
  const bool use_lb = (p.flags & kLowerBound) != 0;
  const float Ah = __expf(hr.alog);
  auto f = [&](uint32_t raw) {
    return __uint_as_float(kg_bf16 ? raw << 16 : raw);
  };
#pragma unroll
  for (int jj = 0; jj < C::JG; ++jj) {
    const int j = tid + jj * C::NT;
    const int t = j / D, k = j % D;
    if (t < QMAX) {
      const bool ok = t < n;
      fs.cT[k][t] = pr.cv[jj];
      fs.w[t][k] = ok ? f(pr.kr[jj]) : 0.0f;
      fs.dec[t][k] =
          ok ? __expf(kda_gate(f(pr.gr[jj]) + hr.gb[jj], Ah, use_lb, p.lb))
             : 1.0f;
    }
  }
  lds_barrier();
  for (int t = wave; t < QMAX; t += C::NT / 64) {
    float x = 0.0f;
    for (int c = lane; c < D; c += 64) x += fs.w[t][c] * fs.w[t][c];
    const float tot = wave_sum(x);
    if (lane == 0) fs.ksum[t] = tot;
  }
  lds_barrier();
  if (tid < D) {
    float suf = 1.0f;
#pragma unroll
    for (int t = QMAX - 1; t >= 0; --t) {
      if (t < n) {
        fs.w[t][tid] *= rsqrtf(fs.ksum[t] + kNormEps) * suf;
        suf *= fs.dec[t][tid];
      }
    }
    fs.gam[tid] = suf;
  }
  lds_barrier();
}

// S <- S diag(Gam) + sum_{t<n} c_t w_t^T on the register tile, written back
// to the checkpoint slot.
template <int D, int QMAX>
__device__ __forceinline__ void flush_fold(const VerifyParams& p,
                                           const FlushSmem<D, QMAX, true>& fs,
                                           const Item& it, int n,
                                           Tile<D, QMAX>& st) {
  using C = VerifyCfg<D, QMAX>;
  const int tid = fresh_tid();
  const int lg = tid % C::L, rg = tid / C::L;
  float* dst = const_cast<float*>(p.state) + int64_t(it.slot) * p.s_slot +
               int64_t(it.h) * D * D;
  // Column chunk outer, position inner, the tile updated in place: one
  // column vector and one correction per pass are live at a time (the
  // operations per element are the same, in the same order).
#pragma unroll
  for (int c = 0; c < C::CHUNKS; ++c) {
    const int col = c * 4 * C::L + 4 * lg;
    const f4 g4 = *reinterpret_cast<const f4*>(&fs.gam[col]);
#pragma unroll
    for (int pp = 0; pp < C::PASSES; ++pp) st[pp][c] = st[pp][c] * g4;
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      if (t < n) {
        const f4 w4 = *reinterpret_cast<const f4*>(&fs.w[t][col]);
#pragma unroll
        for (int pp = 0; pp < C::PASSES; ++pp) {
          const float cv = fs.cT[pp * C::RPP + rg][t];
          f4& a = st[pp][c];
          a.x = fmaf(cv, w4.x, a.x);
          a.y = fmaf(cv, w4.y, a.y);
          a.z = fmaf(cv, w4.z, a.z);
          a.w = fmaf(cv, w4.w, a.w);
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < C::PASSES; ++pp)
      st_stream(dst + (pp * C::RPP + rg) * D + col, st[pp][c]);
  }
}

// The deferred flush of an item whose slot is live but whose window is
// empty (q = 0): the pending positions are still folded into the checkpoint
// and written back; nothing else is read or written.
template <int D, int QMAX>
__device__ __forceinline__ void flush_only_item(const VerifyParams& p,
                                                FlushSmem<D, QMAX, true>& fs,
                                                const Item& it) {
  using C = VerifyCfg<D, QMAX>;
  if (!it.rec_ok) return;
  const int n = min(max(sload1(p.pending + it.b), 0), p.Q);
  if (n == 0) return;
  const int tid = fresh_tid();
  HeadRegs<D, QMAX> hr;
  load_head<D, QMAX>(p, it.h, hr);
  PendingRegs<D, QMAX> pr;
  load_pending<D, QMAX>(p, it, n, pr);
  const int lg = tid % C::L, rg = tid / C::L;
  const float* __restrict__ sbase =
      p.state + int64_t(it.slot) * p.s_slot + int64_t(it.h) * D * D;
  Tile<D, QMAX> st;
#pragma unroll
  for (int pp = 0; pp < C::PASSES; ++pp)
#pragma unroll
    for (int c = 0; c < C::CHUNKS; ++c)
      st[pp][c] = ld_stream(sbase + (pp * C::RPP + rg) * D + c * 4 * C::L +
                            4 * lg);
  flush_prepare<D, QMAX>(p, fs, n, pr, hr);
  flush_fold<D, QMAX>(p, fs, it, n, st);
}

// Null block (null or out-of-pool slot): +0.0 outputs, no state, record or
// conv byte touched.
template <int D, int QMAX>
__device__ __forceinline__ void null_item(const VerifyParams& p,
                                          const Item& it) {
  using C = VerifyCfg<D, QMAX>;
  for (int j = fresh_tid(); j < it.q * D; j += C::NT) {
    const int t = j / D, v = j - t * D;
    st_elem(p.out, int64_t(it.bos + t) * p.s_out + int64_t(it.h) * D + v,
            0.0f, (p.flags & kOutBf16) != 0);
  }
}

// One live item, loads issued here (one-workgroup-per-item and ticket
// schedules).  `drawn` is thread 0's freshly drawn ticket; it is published
// through LDS at the first barrier, after which `advance()` starts the
// scalar loads of the next item's metadata.
// DV < D: one V-tile of the item (rows it.v0 .. it.v0 + DV); `advance()`
// then performs its arrival (see kda_verify_vtile_kernel) and LDS
// ticket[1] says, from the next barrier on, whether this V-tile rolls the
// q and k channels.
template <int D, int QMAX, bool ACT_BF16, bool FULL, bool FLUSH,
          bool PERSISTENT, int DV = D, class Advance>
__device__ __forceinline__ void verify_item(const VerifyParams& p,
                                            VerifySmem<D, QMAX>& sm,
                                            FlushSmem<D, QMAX, FLUSH>& fs,
                                            const Item& it, int drawn,
                                            int buf, Advance&& advance) {
  using C = VerifyCfg<D, QMAX, DV>;
  using AT = typename Act<ACT_BF16>::T;
  static_assert(DV == D || !(FLUSH || PERSISTENT), "V-tiles: plain verify");
  const int tid = threadIdx.x;
  const int h = it.h;
  const int q = FULL ? QMAX : it.q;
  const int HD = p.H * D;
  const int v0 = DV == D ? 0 : it.v0;
  // small loads first (vector-memory counters retire in issue order)
  HeadRegs<D, QMAX, DV> hr;
  load_head<D, QMAX, DV>(p, h, hr, v0);
  // deferred flush: positions still pending in the record row
  int n_pend = 0;
  PendingRegs<D, QMAX> pr;
  if constexpr (FLUSH) {
    if (it.rec_ok) n_pend = min(max(sload1(p.pending + it.b), 0), p.Q);
    if (n_pend > 0) load_pending<D, QMAX>(p, it, n_pend, pr);
  }
  Small<D, QMAX, ACT_BF16, DV> s;
  {
    const AT* __restrict__ xq =
        static_cast<const AT*>(p.mixed_qkv) + int64_t(it.bos) * p.s_x;
    const AT* __restrict__ cs =
        static_cast<const AT*>(p.conv_state) + int64_t(it.slot) * p.s_cs_slot;
    const AT* __restrict__ graw = static_cast<const AT*>(p.raw_gate) +
                                  int64_t(it.bos) * p.s_g + h * D;
    const AT* __restrict__ rbeta = static_cast<const AT*>(p.raw_beta) +
                                   int64_t(it.bos) * p.s_beta + h;
    const int s_cc = p.s_cs_chan, s_ct = p.s_cs_tok;
#pragma unroll
    for (int jj = 0; jj < C::JC; ++jj) {
      const int j = tid + jj * C::NT;
      if (j < C::NCONV) {
        int part, d;
        conv_slot<D, DV>(j, v0, part, d);
        const int ch = part * HD + h * D + d;
        if (p.flags & kNoConv) {
          // q | k | v given after the convolution: no history
#pragma unroll
          for (int i = 0; i < 3; ++i) s.hist[jj][i] = AT{};
        } else if (p.flags & kConvRow) {
          const uint32_t* rp = reinterpret_cast<const uint32_t*>(cs + ch * s_cc);
#pragma unroll
          for (int i = 0; i < Small<D, QMAX, ACT_BF16, DV>::RD; ++i)
            s.row[jj][i] = rp[i];
        } else {
          const int co = ch * s_cc + (it.a - 1) * s_ct;
#pragma unroll
          for (int i = 0; i < 3; ++i) s.hist[jj][i] = cs[co + i * s_ct];
        }
#pragma unroll
        for (int t = 0; t < QMAX; ++t)
          if (t < q) s.xs[jj][t] = xq[t * p.s_x + ch];
      }
    }
#pragma unroll
    for (int jj = 0; jj < C::JG; ++jj) {
      const int j = tid + jj * C::NT;
      const int t = j / D, k = j - t * D;
      if (t < q) s.gv[jj] = graw[t * p.s_g + k];
    }
    // One workgroup per item: loaded by every lane (from a clamped, always
    // valid position) rather than under `tid < q`.  A conditional load lets
    // the compiler merge the sigmoid into its block, which then waits for
    // every small load before the state tile is issued.  (The persistent
    // loop keeps the conditional form: the other one costs it scalar
    // registers, and it is not the default schedule.)
    if constexpr (PERSISTENT) {
      s.bv = AT{};
      if (tid < q) s.bv = rbeta[tid * p.s_beta];
    } else {
      s.bv = rbeta[min(tid, q - 1) * p.s_beta];
    }
  }
  // the state tile, in two halves (the second once the conv registers are
  // free)
  const int lg = tid % C::L, rg = tid / C::L;
  const float* __restrict__ sbase = p.state + int64_t(it.slot) * p.s_slot +
                                   int64_t(h) * D * D + v0 * D;
  constexpr int P0 = (C::PASSES + 1) / 2;
  Tile<D, QMAX, DV> st;
#pragma unroll
  for (int pp = 0; pp < P0; ++pp)
#pragma unroll
    for (int c = 0; c < C::CHUNKS; ++c)
      st[pp][c] = ld_stream(sbase + (pp * C::RPP + rg) * D + c * 4 * C::L +
                            4 * lg);
  // the pending records are read (and their LDS views built) before phase
  // 0 writes this step's records into the same row
  if constexpr (FLUSH) {
    if (n_pend > 0) flush_prepare<D, QMAX>(p, fs, n_pend, pr, hr);
  }
  item_front<D, QMAX, ACT_BF16, FULL, DV, DV == D>(p, sm, it, s, hr, [&] {
#pragma unroll
    for (int pp = P0; pp < C::PASSES; ++pp)
#pragma unroll
      for (int c = 0; c < C::CHUNKS; ++c)
        st[pp][c] = ld_stream(sbase + (pp * C::RPP + rg) * D +
                              c * 4 * C::L + 4 * lg);
  });
  if (tid == 0) sm.ticket[buf ^ 1] = drawn;
  lds_barrier();
  // Metadata of the next item: scalar loads in flight from here on.
  advance();
  item_back<D, QMAX, FULL, DV, PERSISTENT>(p, sm, it, st,
                                           [&](Tile<D, QMAX, DV>& t) {
    if constexpr (FLUSH) {
      if (n_pend > 0) flush_fold<D, QMAX>(p, fs, it, n_pend, t);
    }
    if constexpr (DV != D) {
      // the last V-tile to arrive rolls the q and k channels
      if ((p.flags & kNoConv) == 0 && sm.ticket[1] != 0)
        roll_qk<D, QMAX, ACT_BF16, FULL, DV>(p, it, s);
    }
  });
}

template <int D, int QMAX, bool ACT_BF16>
__global__ void __launch_bounds__((VerifyCfg<D, QMAX>::NT),
                                  (VerifyCfg<D, QMAX>::TICKET_MIN_WAVES))
    kda_verify_kernel(VerifyParams p) {
  using C = VerifyCfg<D, QMAX>;
  __shared__ VerifySmem<D, QMAX> sm;
  FlushSmem<D, QMAX, false> nofs;
  const int tid = threadIdx.x;
  // Ticket protocol: a ticket claims per_ticket consecutive items.  Every
  // workgroup draws tickets until one is past the last, drawing the next
  // ticket while it works on the last item of its current chunk.  Exactly
  // n_tickets + gridDim.x draws happen in total, so the draw that returns
  // the largest value is the last one; its workgroup resets the counter for
  // the next launch on the stream.
  if (tid == 0) sm.ticket[0] = atomicAdd(p.counter, 1);
  lds_barrier();
  int ticket = uniform(sm.ticket[0]);
  int item = ticket * p.per_ticket;
  int end = min(item + p.per_ticket, p.n_items);
  Item it{};
  if (ticket < p.n_tickets) it = load_item(p, uniform(item / p.H), uniform(item % p.H));
  int buf = 0;
  while (ticket < p.n_tickets) {
    const bool last = item + 1 >= end;
    int drawn = 0;
    if (last && tid == 0) drawn = atomicAdd(p.counter, 1);
    int nticket = ticket, nitem = item + 1, nend = end;
    Item nx{};
    auto advance = [&]() {
      if (last) {
        nticket = uniform(sm.ticket[buf ^ 1]);
        nitem = nticket * p.per_ticket;
        nend = min(nitem + p.per_ticket, p.n_items);
      }
      if (nticket < p.n_tickets) nx = load_item(p, uniform(nitem / p.H),
                                                 uniform(nitem % p.H));
    };
    if (it.live) {
      if (it.q == QMAX)
        verify_item<D, QMAX, ACT_BF16, true, false, true>(p, sm, nofs, it, drawn,
                                                    buf, advance);
      else
        verify_item<D, QMAX, ACT_BF16, false, false, true>(p, sm, nofs, it, drawn,
                                                     buf,
                                              advance);
    } else {
      // Null block: zero outputs, touch no state, record or conv byte.
      for (int j = tid; j < it.q * D; j += C::NT) {
        const int t = j / D, v = j - t * D;
        st_elem(p.out, int64_t(it.bos + t) * p.s_out + int64_t(it.h) * D + v,
                0.0f, (p.flags & kOutBf16) != 0);
      }
      if (tid == 0) sm.ticket[buf ^ 1] = drawn;
    }
    lds_barrier();
    if (!it.live) advance();
    buf ^= 1;
    ticket = nticket;
    item = nitem;
    end = nend;
    it = nx;
  }
  if (tid == 0 && ticket == p.n_tickets + int(gridDim.x) - 1)
    atomicExch(p.counter, 0);
}

// One workgroup per (head, request) item on a (head, request) grid; the
// hardware dispatcher refills each compute unit as workgroups retire (which
// also balances ragged windows).  No loop-carried state, no ticket counter.
// FLUSH: the deferred flush of pending record positions comes first.
template <int D, int QMAX, bool ACT_BF16, bool FLUSH>
__global__ void __launch_bounds__((VerifyCfg<D, QMAX>::NT),
                                  (VerifyCfg<D, QMAX>::MIN_WAVES))
    kda_verify_grid_kernel(VerifyParams p) {
  using C = VerifyCfg<D, QMAX>;
  __shared__ VerifySmem<D, QMAX> sm;
  __shared__ FlushSmem<D, QMAX, FLUSH> fs;
  // XCD-aware order: the dispatcher hands consecutive workgroups to the 8
  // XCDs in turn, so workgroup i takes item (i mod 8) * n/8 + i/8 and each
  // XCD works through one contiguous eighth of the (request, head) items
  // (4% faster for the fused flush at 1024 requests, neutral otherwise).
  const int n = p.B * p.H;
  const int lin = int(blockIdx.x) + p.H * int(blockIdx.y);
  const int item = (n & 7) == 0 ? (lin & 7) * (n >> 3) + (lin >> 3) : lin;
  const int ib = item / p.H;
  const Item it = load_item(p, uniform(ib), uniform(item - ib * p.H));
  auto advance = [] {};
  if (it.live) {
    if (it.q == QMAX)
      verify_item<D, QMAX, ACT_BF16, true, FLUSH, false>(p, sm, fs, it, 0, 0,
                                                  advance);
    else
      verify_item<D, QMAX, ACT_BF16, false, FLUSH, false>(p, sm, fs, it, 0, 0,
                                                   advance);
  } else if (FLUSH && it.slot_ok) {
    // live slot, empty window: only the deferred flush
    if constexpr (FLUSH) flush_only_item<D, QMAX>(p, fs, it);
  } else {
    // Null block: zero outputs, touch no state, record or conv byte.
    for (int j = threadIdx.x; j < it.q * D; j += C::NT) {
      const int t = j / D, v = j - t * D;
      st_elem(p.out, int64_t(it.bos + t) * p.s_out + int64_t(it.h) * D + v,
              0.0f, (p.flags & kOutBf16) != 0);
    }
  }
}

// One workgroup per (request, head, V-tile): each of the VT = D / DV
// workgroups of a (request, head) item verifies DV rows of its state (the
// ops page launches its verify on a (V-blocks, requests, heads) grid), for
// batches too small to fill the GPU with whole items.  Every V-tile computes
// the conv of the head's q and k channels (all of them feed its column
// phase) and of its own value channels, which it also rolls.  The q and k
// channels are rolled once, by the last V-tile of the item to have read
// their history: after the barrier that follows phase 0 (every thread of
// the workgroup has used its loaded history by then), thread 0 adds 1 to
// the item's arrival counter work_counter[1 + b * H + h]; the V-tile that
// sees VT - 1 sets it back to 0 and rolls them.  Results are bitwise those
// of kda_verify_grid_kernel.
template <int D, int QMAX, bool ACT_BF16, int DV>
__global__ void __launch_bounds__((VerifyCfg<D, QMAX, DV>::NT),
                                  (VerifyCfg<D, QMAX, DV>::MIN_WAVES))
    kda_verify_vtile_kernel(VerifyParams p) {
  using C = VerifyCfg<D, QMAX, DV>;
  constexpr int VT = D / DV;
  __shared__ VerifySmem<D, QMAX> sm;
  FlushSmem<D, QMAX, false> nofs;
  // XCD-aware order over (request, head, V-tile) with the V-tile fastest,
  // so that the V-tiles of one item share an XCD's L2 (they all read the
  // item's q and k inputs)
  const int n = p.B * p.H * VT;
  const int lin = int(blockIdx.x);
  const int item = (n & 7) == 0 ? (lin & 7) * (n >> 3) + (lin >> 3) : lin;
  const int bh = item / VT;
  const int ib = bh / p.H;
  Item it = load_item(p, uniform(ib), uniform(bh - ib * p.H));
  it.v0 = uniform(item - bh * VT) * DV;
  int* __restrict__ arrive = p.counter + 1 + bh;
  // Arrival (right after the phase-0 barrier).  The increment is read back
  // from LDS, where thread 0 stored it before the barrier, so the atomic
  // cannot be issued before every wave has passed that barrier.
  auto advance = [&] {
    if (threadIdx.x == 0 && (p.flags & kNoConv) == 0) {
      const int inc = sm.ticket[0];
      const int old = atomicAdd(arrive, inc);
      const int last = old == VT - 1 ? 1 : 0;
      if (last)
        __hip_atomic_store(arrive, 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      sm.ticket[1] = last;
    }
  };
  if (it.live) {
    // drawn = 1 with buf = 1: thread 0 stores the increment 1 in ticket[0]
    if (it.q == QMAX)
      verify_item<D, QMAX, ACT_BF16, true, false, false, DV>(p, sm, nofs, it,
                                                             1, 1, advance);
    else
      verify_item<D, QMAX, ACT_BF16, false, false, false, DV>(p, sm, nofs, it,
                                                              1, 1, advance);
  } else {
    // Null block: zero this V-tile's outputs, touch nothing else.
    for (int j = threadIdx.x; j < it.q * DV; j += C::NT) {
      const int t = j / DV, v = it.v0 + (j - t * DV);
      st_elem(p.out, int64_t(it.bos + t) * p.s_out + int64_t(it.h) * D + v,
              0.0f, (p.flags & kOutBf16) != 0);
    }
  }
}

// Workgroups of `kern` resident on the current device at once (cached per
// device: the value does not change during the process).
template <class K>
int resident_grid(K kern, int threads, int* cache, int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return 0;
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(kern), threads, 0);
  if (e != hipSuccess) return int(e);
  *out = max(1, cus * max(per_cu, 1));
  if (dev >= 0 && dev < 64) cache[dev] = *out;
  return 0;
}

// V-tiles of a head with D rows: VT = 2, 4 or 8 (head dims 64 and 128,
// windows up to 8).
template <int D, int QMAX, bool ACT_BF16>
int launch_vtiles(const VerifyParams& p, int vt, hipStream_t stream) {
  if constexpr ((D == 64 || D == 128) && QMAX <= 8) {
    const int64_t n = int64_t(p.B) * p.H * vt;
    if (n > 0x7fffffff) return int(hipErrorInvalidConfiguration);
    switch (vt) {
      case 2:
        launch_kernel((kda_verify_vtile_kernel<D, QMAX, ACT_BF16, D / 2>),
                      dim3(unsigned(n)),
                      dim3(VerifyCfg<D, QMAX, D / 2>::NT), 0, stream, p);
        return int(hipGetLastError());
      case 4:
        launch_kernel((kda_verify_vtile_kernel<D, QMAX, ACT_BF16, D / 4>),
                      dim3(unsigned(n)),
                      dim3(VerifyCfg<D, QMAX, D / 4>::NT), 0, stream, p);
        return int(hipGetLastError());
      case 8:
        launch_kernel((kda_verify_vtile_kernel<D, QMAX, ACT_BF16, D / 8>),
                      dim3(unsigned(n)),
                      dim3(VerifyCfg<D, QMAX, D / 8>::NT), 0, stream, p);
        return int(hipGetLastError());
      default:
        return int(hipErrorInvalidValue);
    }
  }
  return int(hipErrorInvalidValue);
}

template <int D, int QMAX, bool ACT_BF16>
int launch_one(const VerifyParams& p, int schedule, int grid,
               hipStream_t stream) {
  using C = VerifyCfg<D, QMAX>;
  // One workgroup per item is the default: on gfx950 the hardware
  // dispatcher balances ragged windows by itself and the per-item kernel
  // carries no loop state, which the ticket loop pays for in registers.
  if (p.pending != nullptr) {  // the deferred flush: per-item kernel only
    if (p.B > 65535) return int(hipErrorInvalidConfiguration);
    launch_kernel((kda_verify_grid_kernel<D, QMAX, ACT_BF16, true>),
                  dim3(p.H, p.B), dim3(C::NT), 0, stream, p);
    return int(hipGetLastError());
  }
  if (schedule == kScheduleVTiles && p.v_tiles > 1)
    return launch_vtiles<D, QMAX, ACT_BF16>(p, p.v_tiles, stream);
  if (schedule != kScheduleTickets && p.B <= 65535) {
    launch_kernel((kda_verify_grid_kernel<D, QMAX, ACT_BF16, false>),
                  dim3(p.H, p.B), dim3(C::NT), 0, stream, p);
    return int(hipGetLastError());
  }
  // Tickets (also for more requests than a grid row holds).
  auto kern = kda_verify_kernel<D, QMAX, ACT_BF16>;
  if (grid <= 0) {
    static int cache[64];
    const int e = resident_grid(kern, C::NT, cache, &grid);
    if (e != 0) return e;
  }
  if (p.counter == nullptr) return int(hipErrorInvalidValue);
  VerifyParams q = p;
  if (q.per_ticket <= 0) q.per_ticket = 1;
  q.n_tickets = (q.n_items + q.per_ticket - 1) / q.per_ticket;
  grid = min(grid, q.n_tickets);
  launch_kernel(kern, dim3(grid), dim3(C::NT), 0, stream, q);
  return int(hipGetLastError());
}

template <int D, bool ACT_BF16>
int launch_q(const VerifyParams& p, int sched, int grid, hipStream_t stream) {
  if (p.Q <= 4) return launch_one<D, 4, ACT_BF16>(p, sched, grid, stream);
  if (p.Q <= 8) return launch_one<D, 8, ACT_BF16>(p, sched, grid, stream);
  return launch_one<D, 16, ACT_BF16>(p, sched, grid, stream);
}

}  // namespace
}  // namespace kda
