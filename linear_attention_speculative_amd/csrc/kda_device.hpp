// Device-side helpers for the gfx950 KDA RecoverSSM kernels: bf16
// conversion, cross-lane reductions with DPP, an LDS-only workgroup barrier,
// streaming 16-byte memory ops and the KDA gate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef float f4 __attribute__((ext_vector_type(4)));

// ---- element conversion ------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// fp32 -> bf16 with round-to-nearest-even; NaNs stay NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ float ld_elem(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i])
              : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void st_elem(void* p, int64_t i, float v,
                                        bool bf16) {
  if (bf16)
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else
    static_cast<float*>(p)[i] = v;
}

template <bool BF16>
struct Act;
template <>
struct Act<true> {
  typedef uint16_t T;
  static __device__ __forceinline__ float f(T x) { return bf16_to_f32(x); }
};
template <>
struct Act<false> {
  typedef float T;
  static __device__ __forceinline__ float f(T x) { return x; }
};

// ---- addressing ------------------------------------------------------------------

// Element `off` of a wave-uniform base pointer, with the offset taken as an
// unsigned 32-bit byte count (the host checks that every in-item offset
// fits).  Written this way the compiler can use the scalar-base + 32-bit
// vector-offset form of global memory instructions, which keeps one VGPR
// per address instead of two.
template <class T>
__device__ __forceinline__ T& at(T* base, uint32_t off) {
  using C = typename std::conditional<std::is_const<T>::value, const char,
                                      char>::type;
  return *reinterpret_cast<T*>(reinterpret_cast<C*>(base) +
                               off * uint32_t(sizeof(T)));
}

// A device address held as an integer (the per-layer address tables of the
// commit) as a pointer known to point to global memory.  Going through the
// global address space lets the compiler emit global memory instructions
// for everything derived from it; a plain integer-to-pointer cast gives a
// generic pointer and flat instructions, which also count against the LDS
// wait counter, so that every LDS wait (a barrier) would wait for the
// streaming loads as well.
template <class T>
__device__ __forceinline__ T* global_addr(int64_t a) {
  return (T*)(__attribute__((address_space(1))) T*)(uintptr_t)a;
}

// Scalar loads of values the kernel never writes (per-request metadata,
// per-head parameters) at wave-uniform addresses, with their own wait.
// Written out because inside a persistent loop that also stores to global
// memory the compiler cannot prove these locations unclobbered and would
// use vector loads, whose completion waits (in order) behind the state tile
// streaming in for the next item.  All addresses must be 4-byte aligned.
// A pointer the compiler must keep in scalar registers (an inline-asm "s"
// operand is not moved out of vector registers by itself).
__device__ __forceinline__ const int32_t* sgpr_ptr(const int32_t* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  return reinterpret_cast<const int32_t*>((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ void sload4(const int32_t* a0, const int32_t* a1,
                                       const int32_t* a2, const int32_t* a3,
                                       int32_t& v0, int32_t& v1, int32_t& v2,
                                       int32_t& v3) {
  a0 = sgpr_ptr(a0);
  a1 = sgpr_ptr(a1);
  a2 = sgpr_ptr(a2);
  a3 = sgpr_ptr(a3);
  asm volatile(
      "s_load_dword %0, %4, 0x0\n\t"
      "s_load_dword %1, %5, 0x0\n\t"
      "s_load_dword %2, %6, 0x0\n\t"
      "s_load_dword %3, %7, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      // early-clobber: a result register must not alias an address that a
      // later load of the sequence still reads
      : "=&s"(v0), "=&s"(v1), "=&s"(v2), "=&s"(v3)
      : "s"(a0), "s"(a1), "s"(a2), "s"(a3)
      : "memory");
}

__device__ __forceinline__ int32_t sload1(const int32_t* a0) {
  a0 = sgpr_ptr(a0);
  int32_t v0;
  asm volatile(
      "s_load_dword %0, %1, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v0)
      : "s"(a0)
      : "memory");
  return v0;
}

// ---- streaming 16-byte accesses (state rows are touched once) -----------------

__device__ __forceinline__ f4 ld_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ void st_stream(float* p, f4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}

// ---- synchronisation ---------------------------------------------------------

// Workgroup barrier that orders LDS only.  Outstanding global loads (the
// prefetched state tile) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- cross-lane reductions ----------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// DPP control words (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <- 7-i within 8
constexpr int kRowMirror = 0x140;      // lane i <- 15-i within 16

// Sum over aligned groups of G consecutive lanes; every lane of a group
// receives the group total.  Groups up to 16 use DPP only; 32 adds a
// swizzle across the two halves of each 32-lane half-wave.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32,
                "group size");
  if constexpr (G >= 2) v += dpp<kQuadXor1>(v);
  if constexpr (G >= 4) v += dpp<kQuadXor2>(v);
  if constexpr (G >= 8) v += dpp<kRowHalfMirror>(v);
  if constexpr (G >= 16) v += dpp<kRowMirror>(v);
  if constexpr (G >= 32)
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v),
                                                    0x401F));  // xor 16
  return v;
}

// Value of the partner lane at distance S inside a 16-lane row, for the
// pairings used by transpose_sum (each pairs lanes that differ in bit S).
template <int S>
__device__ __forceinline__ float partner(float v) {
  static_assert(S == 1 || S == 2 || S == 4 || S == 8, "stride");
  if constexpr (S == 8) return dpp<kRowMirror>(v);
  if constexpr (S == 4) return dpp<kRowHalfMirror>(v);
  if constexpr (S == 2) return dpp<kQuadXor2>(v);
  return dpp<kQuadXor1>(v);
}

// Transposing reduction over aligned groups of G lanes (G <= 16): every lane
// holds N partial values (N <= G, powers of two); afterwards lane j of a
// group holds the group total of value index j >> (log2 G - log2 N).  Each
// halving step keeps one half of the values and adds the partner's copy of
// that half, so N values cost N - 1 adds instead of N log2 G.
template <int S, int NLIVE, int N>
__device__ __forceinline__ void transpose_step(float (&v)[N], int j) {
  if constexpr (S >= 1) {
    if constexpr (NLIVE > 1) {
      const bool upper = (j & S) != 0;
#pragma unroll
      for (int k = 0; k < NLIVE / 2; ++k) {
        const float keep = upper ? v[k + NLIVE / 2] : v[k];
        const float send = upper ? v[k] : v[k + NLIVE / 2];
        v[k] = keep + partner<S>(send);
      }
      transpose_step<S / 2, NLIVE / 2>(v, j);
    } else {
      v[0] += partner<S>(v[0]);
      transpose_step<S / 2, 1>(v, j);
    }
  }
}

template <int G, int N>
__device__ __forceinline__ float transpose_sum(float (&v)[N], int j) {
  static_assert(G >= 1 && G <= 16 && N >= 1 && N <= G, "sizes");
  transpose_step<G / 2, N>(v, j);
  return v[0];
}

// Sum over the whole 64-lane wave, returned as a wave-uniform value.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  const int b = __float_as_int(v);
  return __int_as_float(__builtin_amdgcn_readlane(b, 0)) +
         __int_as_float(__builtin_amdgcn_readlane(b, 16)) +
         __int_as_float(__builtin_amdgcn_readlane(b, 32)) +
         __int_as_float(__builtin_amdgcn_readlane(b, 48));
}

// threadIdx.x as a value the compiler must treat as new at every call.
// Inside a persistent loop, lane offsets derived from it would otherwise be
// hoisted out of the loop and kept live (or spilled) across it; recomputing
// them per item costs a few instructions.
__device__ __forceinline__ int fresh_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  // the range survives the opaque copy: divisions by powers of two then
  // need no sign fix-up (a value the compiler otherwise keeps, or spills)
  __builtin_assume(t >= 0 && t < 1024);
  return t;
}

__device__ __forceinline__ int uniform(int x) {
  return __builtin_amdgcn_readfirstlane(x);
}

// ---- KDA math -------------------------------------------------------------------

// Hardware reciprocal (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float rcp_(float x) {
  return __builtin_amdgcn_rcpf(x);
}

__device__ __forceinline__ float sigmoidf_(float x) {
  return rcp_(1.0f + __expf(-x));
}

// Log-decay of one channel from x = raw gate + dt_bias and A = exp(A_log):
// bounded form lb * sigmoid(A x), else -A * softplus(x) where softplus is the
// identity above 20 (ops page, `_kda_gate`).  ln(1 + e^x) loses its low bits
// for very negative x, where it is below 1e-7 and the decay rounds to 1.
__device__ __forceinline__ float kda_gate(float x, float A, bool use_lb,
                                          float lb) {
  if (use_lb) return lb * sigmoidf_(A * x);
  const float sp = x > 20.0f ? x : __logf(1.0f + __expf(x));
  return -A * sp;
}

constexpr float kNormEps = 1e-6f;  // inside the square root of both norms

}  // namespace kda
