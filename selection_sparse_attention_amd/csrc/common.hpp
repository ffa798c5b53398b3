// Device helpers shared by the gfx950 kernels: element access, order-keys
// for radix selection, wave/block reductions, and launch argument structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- elements
// bf16 values are handled as raw 16-bit patterns: widening is a shift, and
// narrowing rounds to nearest even.
struct bf16_t { uint16_t v; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);   // round to nearest, ties to even
  return uint16_t(u >> 16);
}

// Round a double once to the nearest bf16 (ties to even), for normal values
// in range: the low 45 bits of the double's significand are rounded away.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  uint64_t u = __double_as_longlong(x);
  u += 0x0FFFFFFFFFFFull + ((u >> 45) & 1ull);
  u &= ~0x1FFFFFFFFFFFull;
  return uint16_t(__float_as_uint((float)__longlong_as_double(u)) >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int bytes = 2;
  __device__ static float load(const void* p, int64_t i) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  }
  __device__ static void store(void* p, int64_t i, float x) {
    reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
  }
  __device__ static void store_d(void* p, int64_t i, double x) {
    reinterpret_cast<uint16_t*>(p)[i] = f64_to_bf16(x);
  }
};
template <> struct Elem<float> {
  static constexpr int bytes = 4;
  __device__ static float load(const void* p, int64_t i) {
    return reinterpret_cast<const float*>(p)[i];
  }
  __device__ static void store(void* p, int64_t i, float x) {
    reinterpret_cast<float*>(p)[i] = x;
  }
  __device__ static void store_d(void* p, int64_t i, double x) {
    reinterpret_cast<float*>(p)[i] = (float)x;
  }
};

typedef uint32_t vl_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t vl_u32x4 __attribute__((ext_vector_type(4)));
typedef float vl_f32x2 __attribute__((ext_vector_type(2)));
typedef float vl_f32x4 __attribute__((ext_vector_type(4)));

// A plain load, or a non-temporal one (streamed data read once: it does not
// displace reused lines in the caches).
template <bool NT, typename V>
__device__ __forceinline__ V vl_load(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Load N consecutive elements starting at element offset i (16-byte chunks;
// the caller guarantees alignment) and widen them to fp32.
template <typename T, int N, bool NT = false> struct VecLoad;
template <int N, bool NT> struct VecLoad<bf16_t, N, NT> {
  static_assert(N % 8 == 0 || N == 4, "bf16 vector loads are 8 or 4 elements");
  __device__ static void run(const void* base, int64_t i, float* out) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + i;
    if constexpr (N == 4) {
      const vl_u32x2 w = vl_load<NT>(reinterpret_cast<const vl_u32x2*>(p));
      out[0] = bf16_lo(w[0]); out[1] = bf16_hi(w[0]);
      out[2] = bf16_lo(w[1]); out[3] = bf16_hi(w[1]);
    } else {
#pragma unroll
      for (int c = 0; c < N / 8; ++c) {
        const vl_u32x4 w = vl_load<NT>(reinterpret_cast<const vl_u32x4*>(p + 8 * c));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          out[8 * c + 2 * e] = bf16_lo(w[e]);
          out[8 * c + 2 * e + 1] = bf16_hi(w[e]);
        }
      }
    }
  }
};
template <int N, bool NT> struct VecLoad<float, N, NT> {
  static_assert(N % 4 == 0, "fp32 vector loads are multiples of 4 elements");
  __device__ static void run(const void* base, int64_t i, float* out) {
    const float* p = reinterpret_cast<const float*>(base) + i;
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const vl_f32x4 w = vl_load<NT>(reinterpret_cast<const vl_f32x4*>(p + 4 * c));
      out[4 * c + 0] = w[0]; out[4 * c + 1] = w[1]; out[4 * c + 2] = w[2]; out[4 * c + 3] = w[3];
    }
  }
};

// ---------------------------------------------------------------- order keys
// Monotone map float -> uint32: a > b  <=>  key(a) > key(b) for finite
// values (+0 and -0 are folded to the same key by the caller).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- reductions
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m, int width = kWave) {
  return __shfl_xor(v, m, width);
}

// Workgroup barrier that orders LDS only: the release/acquire fences are
// restricted to the local address space, so the barrier waits for the
// wave's LDS operations but leaves its global loads in flight (a plain
// __syncthreads also drains every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Move a 32- or 64-bit value across lanes with a DPP control (rows outside
// ROWMASK and lanes whose source lies outside the row read 0).
template <int CTRL, int ROWMASK, typename T>
__device__ __forceinline__ T dpp_move(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                             ROWMASK, 0xF, false));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWMASK, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWMASK,
                                                              0xF, false);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4, 8 inside each 16-lane row, then row 0's total broadcast into row 1 and
// row 2 (row_bcast:15), and rows 0-1's total into rows 2-3 (row_bcast:31).
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  v += dpp_move<0x111, 0xF>(v);     // row_shr:1
  v += dpp_move<0x112, 0xF>(v);     // row_shr:2
  v += dpp_move<0x114, 0xF>(v);     // row_shr:4
  v += dpp_move<0x118, 0xF>(v);     // row_shr:8
  v += dpp_move<0x142, 0xA>(v);     // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xC>(v);     // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64),
// using `scratch` (NT/64 entries of T in LDS).  Returns the exclusive value
// and writes the block total to *total.  Its barriers order LDS only, so the
// callers' global loads and stores stay in flight across it.
template <typename T, int NT>
__device__ __forceinline__ T block_exclusive_scan(T v, T* scratch, T* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const T incl = wave_inclusive_scan(v);
  if (lane == 63) scratch[wid] = incl;
  lds_barrier();
  T base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    T s = scratch[w];
    if (w < wid) base += s;
    tot += s;
  }
  lds_barrier();
  *total = tot;
  return base + incl - v;
}

// Agent-scope relaxed atomics used for cross-workgroup counters.
__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agent(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sa
