// Fused short-conv update + RecoverSSM speculative verify of one KDA layer,
// for gfx950 (wave64).  One workgroup handles one (request, head) work item
// at a time and draws items from a ticket counter (persistent grid).
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
// Phases of one item (LDS barriers between them):
//   0  issue the 16-byte streaming loads of the state tile into registers;
//      conv update of the head's 3D channels (history at offset a-1 of the
//      conv state, SiLU), roll the conv state in place, key record; gate
//      decays and the raw-gate half of the key record; sigmoid(beta).
//   1  per column k: partial sums of |k_t|^2, |q_t|^2 and of the pairwise
//      terms <k_s, P_{s,t} k_t>, <k_s, P_{s,t} q_t>; wave reductions.
//   2  norms -> per-column vectors Gam_t k_hat_t, Gam_t q_hat_t (LDS) and the
//      Q x Q coefficient matrices.
//   3  dot products of every state row with the 2Q vectors; group sums over
//      the lanes that share a row (DPP); row results to LDS.
//   4  one thread per row: triangular solve for c_t, outputs o_t; stores of
//      out and of the correction record (coalesced along V).
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

template <int D, int QMAX>
struct VerifyCfg {
  static constexpr int NT = D >= 128 ? 256 : (D == 64 ? 128 : 64);
  // lanes sharing one state row in the dot-product phase
  static constexpr int L =
      D == 128 ? (QMAX <= 8 ? 16 : 32) : (D == 64 ? 16 : (D == 32 ? 8 : 4));
  static constexpr int RPP = NT / L;           // rows per pass
  static constexpr int PASSES = D / RPP;       // passes over the tile
  static constexpr int CHUNKS = D / (4 * L);   // float4 per lane per row
  static constexpr int CW = (D + 63) / 64;     // waves holding columns
  static constexpr int NM = QMAX * (QMAX - 1) / 2;  // <k_s, P k_t>, s < t
  static constexpr int NN = QMAX * (QMAX + 1) / 2;  // <k_s, P q_t>, s <= t
  static constexpr int NV = 2 * QMAX + NM + NN;     // reduced scalars
  static constexpr int DS = 2 * QMAX + 4;           // padded row of dots
  static_assert(RPP * PASSES == D, "tile rows");
  static_assert(CHUNKS * 4 * L == D, "tile columns");
};

template <int D, int QMAX>
struct alignas(16) VerifySmem {
  using C = VerifyCfg<D, QMAX>;
  float y[3][QMAX][D];           // conv outputs q | k | v, positions < q
  float dec[QMAX][D];            // decays d_t
  float vec[2 * QMAX][D];        // Gam_t k_hat_t, then Gam_t q_hat_t
  float dots[D * C::DS];         // per row: S.(Gam k_hat_t), S.(Gam q_hat_t)
  float red[C::CW][C::NV];       // wave partial sums
  float Mc[QMAX][QMAX];          // <k_hat_s, P_{s,t} k_hat_t>, s < t
  float Nc[QMAX][QMAX];          // <k_hat_s, P_{s,t} q_hat_t>, s <= t
  float beta[QMAX];
  int ticket[2];
};

// Index of the pair terms in the reduction vector.
template <int QMAX>
__device__ __forceinline__ constexpr int idx_m(int t, int s) {
  return 2 * QMAX + t * (t - 1) / 2 + s;
}
template <int QMAX>
__device__ __forceinline__ constexpr int idx_n(int t, int s) {
  return 2 * QMAX + QMAX * (QMAX - 1) / 2 + t * (t + 1) / 2 + s;
}

template <int D, int QMAX, bool ACT_BF16>
__device__ __forceinline__ void verify_item(const VerifyParams& p,
                                            VerifySmem<D, QMAX>& sm, int b,
                                            int h) {
  using C = VerifyCfg<D, QMAX>;
  using A = Act<ACT_BF16>;
  using AT = typename A::T;
  const int tid = threadIdx.x;

  // Token rows outside [0, T) are never touched (memory-safety clamp).
  const int bos = p.qsl[b];
  const int q = (bos < 0 || bos >= p.T)
                    ? 0
                    : min(min(max(p.qsl[b + 1] - bos, 0), p.Q), p.T - bos);
  const int slot = p.slots[b];
  if (q == 0) return;
  const int64_t out_col = int64_t(h) * D;
  if (slot <= p.null_id || slot < 0 || slot >= p.N) {
    // Null block: zero outputs, touch no state, record or conv byte.
    for (int j = tid; j < q * D; j += C::NT) {
      const int t = j / D, v = j - t * D;
      st_elem(p.out, int64_t(bos + t) * p.s_out + out_col + v, 0.0f,
              p.out_bf16);
    }
    return;
  }
  const int r = p.record_rows ? p.record_rows[b] : slot;
  const bool rec_ok = r >= 0 && r < p.R;
  const int a = min(max(p.accepted[b], 1), p.Q);

  // ---- phase 0: prefetch the state tile (rows across lane groups) --------
  const int lg = tid % C::L;      // lane within its row group
  const int rg = tid / C::L;      // row group
  const float* sbase =
      p.state + int64_t(slot) * p.s_slot + int64_t(h) * D * D;
  f4 st[C::PASSES][C::CHUNKS];
#pragma unroll
  for (int pp = 0; pp < C::PASSES; ++pp)
#pragma unroll
    for (int c = 0; c < C::CHUNKS; ++c)
      st[pp][c] = ld_stream(sbase + (pp * C::RPP + rg) * D + c * 4 * C::L +
                            4 * lg);

  // ---- phase 0: conv update, roll, key record ------------------------------
  const AT* xq = static_cast<const AT*>(p.mixed_qkv) + int64_t(bos) * p.s_x;
  AT* cs = static_cast<AT*>(p.conv_state) + int64_t(slot) * p.s_cs_slot;
  const int64_t kg_base =
      int64_t(r) * p.s_kg_row + int64_t(h) * p.s_kg_head;
  for (int j = tid; j < 3 * D; j += C::NT) {
    const int part = j / D, d = j - part * D;
    const int64_t ch = int64_t(part) * p.H * D + int64_t(h) * D + d;
    AT* csc = cs + ch * p.s_cs_chan;
    const AT h0 = csc[int64_t(a - 1) * p.s_cs_tok];
    const AT h1 = csc[int64_t(a) * p.s_cs_tok];
    const AT h2 = csc[int64_t(a + 1) * p.s_cs_tok];
    const float w0 = ld_elem(p.conv_weight, ch * p.s_w_chan, p.w_bf16);
    const float w1 = ld_elem(p.conv_weight, ch * p.s_w_chan + p.s_w_tap,
                             p.w_bf16);
    const float w2 = ld_elem(p.conv_weight, ch * p.s_w_chan + 2 * p.s_w_tap,
                             p.w_bf16);
    const float w3 = ld_elem(p.conv_weight, ch * p.s_w_chan + 3 * p.s_w_tap,
                             p.w_bf16);
    AT xs[QMAX];
#pragma unroll
    for (int t = 0; t < QMAX; ++t)
      if (t < q) xs[t] = xq[int64_t(t) * p.s_x + ch];
    float s0 = A::f(h0), s1 = A::f(h1), s2 = A::f(h2);
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      if (t < q) {
        const float s3 = A::f(xs[t]);
        float acc = w0 * s0;
        acc = fmaf(w1, s1, acc);
        acc = fmaf(w2, s2, acc);
        acc = fmaf(w3, s3, acc);
        const float yv = acc * sigmoidf_(acc);
        sm.y[part][t][d] = yv;
        if (part == 1 && rec_ok)
          st_elem(p.key_gate, kg_base + int64_t(t) * p.s_kg_pos + d, yv,
                  p.kg_bf16);
        s0 = s1;
        s1 = s2;
        s2 = s3;
      }
    }
    // Roll: the two newest history entries, then the q new inputs, at the
    // front; positions past 2 + q keep their bytes.
    csc[0] = h1;
    csc[p.s_cs_tok] = h2;
#pragma unroll
    for (int t = 0; t < QMAX; ++t)
      if (t < q) csc[int64_t(2 + t) * p.s_cs_tok] = xs[t];
  }

  // ---- phase 0: gate decays, raw-gate record half, beta ----------------------
  const float Ah = __expf(p.A_log[h]);
  const bool use_lb = p.use_lb != 0;
  const AT* graw = static_cast<const AT*>(p.raw_gate) + int64_t(bos) * p.s_g +
                   int64_t(h) * D;
  for (int j = tid; j < q * D; j += C::NT) {
    const int t = j / D, k = j - t * D;
    const float g0 = A::f(graw[int64_t(t) * p.s_g + k]);
    const float x = g0 + p.dt_bias[int64_t(h) * D + k];
    sm.dec[t][k] = __expf(kda_gate(x, Ah, use_lb, p.lb));
    if (rec_ok)
      st_elem(p.key_gate, kg_base + int64_t(t) * p.s_kg_pos + D + k, g0,
              p.kg_bf16);
  }
  if (tid < q) {
    const AT* rb = static_cast<const AT*>(p.raw_beta);
    sm.beta[tid] = sigmoidf_(A::f(rb[int64_t(bos + tid) * p.s_beta + h]));
  }
  lds_barrier();

  // ---- phase 1: per-column partial sums, reduced per wave --------------------
  const int wave = tid / 64, lane = tid % 64;
  const bool col_ok = tid < D;
  float kk[QMAX], qq[QMAX], dd[QMAX];
#pragma unroll
  for (int t = 0; t < QMAX; ++t) {
    const bool ok = col_ok && t < q;
    kk[t] = ok ? sm.y[1][t][tid] : 0.0f;
    qq[t] = ok ? sm.y[0][t][tid] : 0.0f;
    dd[t] = ok ? sm.dec[t][tid] : 1.0f;
  }
  if (wave < C::CW) {
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      const float s1 = wave_sum(kk[t] * kk[t]);
      const float s2 = wave_sum(qq[t] * qq[t]);
      if (lane == 0) {
        sm.red[wave][t] = s1;
        sm.red[wave][QMAX + t] = s2;
      }
    }
#pragma unroll
    for (int s = 0; s < QMAX; ++s) {
      float P = 1.0f;
#pragma unroll
      for (int t = s; t < QMAX; ++t) {
        if (t > s) {
          P *= dd[t];
          const float m = wave_sum(kk[s] * P * kk[t]);
          if (lane == 0) sm.red[wave][idx_m<QMAX>(t, s)] = m;
        }
        const float n = wave_sum(kk[s] * P * qq[t]);
        if (lane == 0) sm.red[wave][idx_n<QMAX>(t, s)] = n;
      }
    }
  }
  lds_barrier();

  // ---- phase 2: norms, column vectors, coefficient matrices ------------------
  float rk[QMAX], rq[QMAX];
  const float inv_sqrt_d = 1.0f / sqrtf(float(D));
#pragma unroll
  for (int t = 0; t < QMAX; ++t) {
    float sk = 0.0f, sq = 0.0f;
#pragma unroll
    for (int w = 0; w < C::CW; ++w) {
      sk += sm.red[w][t];
      sq += sm.red[w][QMAX + t];
    }
    rk[t] = rsqrtf(sk + kNormEps);
    rq[t] = rsqrtf(sq + kNormEps) * inv_sqrt_d;
  }
  if (col_ok) {
    float gam = 1.0f;
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      gam *= dd[t];
      sm.vec[t][tid] = gam * kk[t] * rk[t];
      sm.vec[QMAX + t][tid] = gam * qq[t] * rq[t];
    }
  }
  for (int j = tid; j < QMAX * QMAX; j += C::NT) {
    const int t = j / QMAX, s = j - t * QMAX;
    float m = 0.0f, n = 0.0f;
#pragma unroll
    for (int w = 0; w < C::CW; ++w) {
      if (s < t) m += sm.red[w][idx_m<QMAX>(t, s)];
      if (s <= t) n += sm.red[w][idx_n<QMAX>(t, s)];
    }
    // rk/rq were computed for every t by every thread above
    float rks = 0.0f, rkt = 0.0f, rqt = 0.0f;
#pragma unroll
    for (int i = 0; i < QMAX; ++i) {
      if (i == s) rks = rk[i];
      if (i == t) {
        rkt = rk[i];
        rqt = rq[i];
      }
    }
    sm.Mc[t][s] = m * rks * rkt;
    sm.Nc[t][s] = n * rks * rqt;
  }
  lds_barrier();

  // ---- phase 3: 2Q dot products per state row --------------------------------
  f4 ka[QMAX][C::CHUNKS], qa[QMAX][C::CHUNKS];
#pragma unroll
  for (int t = 0; t < QMAX; ++t)
#pragma unroll
    for (int c = 0; c < C::CHUNKS; ++c) {
      const int col = c * 4 * C::L + 4 * lg;
      ka[t][c] = *reinterpret_cast<const f4*>(&sm.vec[t][col]);
      qa[t][c] = *reinterpret_cast<const f4*>(&sm.vec[QMAX + t][col]);
    }
#pragma unroll
  for (int pp = 0; pp < C::PASSES; ++pp) {
    float acc[2 * QMAX];
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      float sa = 0.0f, sb = 0.0f;
#pragma unroll
      for (int c = 0; c < C::CHUNKS; ++c) {
        const f4 s4 = st[pp][c];
        sa = fmaf(s4.x, ka[t][c].x, sa);
        sa = fmaf(s4.y, ka[t][c].y, sa);
        sa = fmaf(s4.z, ka[t][c].z, sa);
        sa = fmaf(s4.w, ka[t][c].w, sa);
        sb = fmaf(s4.x, qa[t][c].x, sb);
        sb = fmaf(s4.y, qa[t][c].y, sb);
        sb = fmaf(s4.z, qa[t][c].z, sb);
        sb = fmaf(s4.w, qa[t][c].w, sb);
      }
      acc[t] = group_sum<C::L>(sa);
      acc[QMAX + t] = group_sum<C::L>(sb);
    }
    if (lg == 0) {
      float* drow = &sm.dots[(pp * C::RPP + rg) * C::DS];
#pragma unroll
      for (int i = 0; i < 2 * QMAX; i += 4)
        *reinterpret_cast<f4*>(drow + i) =
            f4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
    }
  }
  lds_barrier();

  // ---- phase 4: per-row triangular solve, outputs and corrections -------------
  if (tid < D) {
    const int v = tid;
    float cc[QMAX];
#pragma unroll
    for (int t = 0; t < QMAX; ++t) {
      if (t < q) {
        float u = sm.dots[v * C::DS + t];
#pragma unroll
        for (int s = 0; s < t; ++s) u = fmaf(sm.Mc[t][s], cc[s], u);
        cc[t] = sm.beta[t] * (sm.y[2][t][v] - u);
        float o = sm.dots[v * C::DS + QMAX + t];
#pragma unroll
        for (int s = 0; s <= t; ++s) o = fmaf(sm.Nc[t][s], cc[s], o);
        st_elem(p.out, int64_t(bos + t) * p.s_out + out_col + v, o,
                p.out_bf16);
        if (rec_ok)
          p.correction[int64_t(r) * p.s_c_row + int64_t(h) * p.s_c_head +
                       int64_t(t) * p.s_c_pos + v] = cc[t];
      }
    }
  }
}

template <int D, int QMAX, bool ACT_BF16>
__global__ void __launch_bounds__((VerifyCfg<D, QMAX>::NT))
    kda_verify_kernel(VerifyParams p) {
  __shared__ VerifySmem<D, QMAX> sm;
  const int tid = threadIdx.x;
  // Ticket protocol: every workgroup draws tickets until one is past the
  // last item, prefetching the next ticket while it works on the current
  // one.  Exactly n_items + gridDim.x draws happen in total, so the draw
  // that returns the largest value is the last one; its workgroup resets
  // the counter for the next launch on the stream.
  if (tid == 0) sm.ticket[0] = atomicAdd(p.counter, 1);
  lds_barrier();
  int ticket = uniform(sm.ticket[0]);
  int buf = 0;
  while (ticket < p.n_items) {
    int next = 0;
    if (tid == 0) next = atomicAdd(p.counter, 1);
    const int b = uniform(ticket / p.H);
    const int h = uniform(ticket - b * p.H);
    verify_item<D, QMAX, ACT_BF16>(p, sm, b, h);
    buf ^= 1;
    if (tid == 0) sm.ticket[buf] = next;
    lds_barrier();
    ticket = uniform(sm.ticket[buf]);
  }
  if (tid == 0 && ticket == p.n_items + int(gridDim.x) - 1)
    atomicExch(p.counter, 0);
}

template <int D, int QMAX, bool ACT_BF16>
int launch_one(const VerifyParams& p, int grid, hipStream_t stream) {
  using C = VerifyCfg<D, QMAX>;
  auto kern = kda_verify_kernel<D, QMAX, ACT_BF16>;
  if (grid <= 0) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                                dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(kern), C::NT, 0);
    if (e != hipSuccess) return int(e);
    grid = max(1, cus * max(per_cu, 1));
  }
  grid = min(grid, p.n_items);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), 0, stream, p);
  return int(hipGetLastError());
}

template <int D, bool ACT_BF16>
int launch_q(const VerifyParams& p, int grid, hipStream_t stream) {
  if (p.Q <= 4) return launch_one<D, 4, ACT_BF16>(p, grid, stream);
  if (p.Q <= 8) return launch_one<D, 8, ACT_BF16>(p, grid, stream);
  return launch_one<D, 16, ACT_BF16>(p, grid, stream);
}

template <bool ACT_BF16>
int launch_d(const VerifyParams& p, int D, int grid, hipStream_t stream) {
  switch (D) {
    case 16: return launch_q<16, ACT_BF16>(p, grid, stream);
    case 32: return launch_q<32, ACT_BF16>(p, grid, stream);
    case 64: return launch_q<64, ACT_BF16>(p, grid, stream);
    case 128: return launch_q<128, ACT_BF16>(p, grid, stream);
    default: return int(hipErrorInvalidValue);
  }
}

__global__ void kda_reset_kernel(int32_t* counter, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) counter[i] = 0;
}

}  // namespace

int launch_verify(const VerifyParams& p, int D, bool act_bf16, int grid,
                  hipStream_t stream) {
  return act_bf16 ? launch_d<true>(p, D, grid, stream)
                  : launch_d<false>(p, D, grid, stream);
}

int launch_reset_counter(int32_t* counter, int n, hipStream_t stream) {
  hipLaunchKernelGGL(kda_reset_kernel, dim3(1), dim3(64), 0, stream, counter,
                     n);
  return int(hipGetLastError());
}

}  // namespace kda
