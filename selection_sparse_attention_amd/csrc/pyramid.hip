// Symmetric mean pyramid over Q, K, V and the parameter-free entry scores
// (Lighthouse summary, Methodology 2A and 2B).
//
// Level 0 is the full-resolution sequence; an entry of level l is the mean of
// p consecutive entries of level l-1, i.e. of its p^l level-0 rows.  Each
// stored coarse entry is that exact mean (accumulated in fp64) rounded once to
// the element type.  The score of a level-0 entry is |q|^2 + |k|^2 (the
// squared l2 norm of the projected query and key: the ranking the norm gives);
// a coarse entry inherits the largest score among the entries it covers.
//
// Each wave streams a run of whole spans (p^(L-1) level-0 rows) of one
// (sequence, head), each lane owning d/64 consecutive dims, in batches of 16
// rows: the next batch's loads are in flight while one is used. The squared
// norms of a batch's rows are summed over the wave together; a level's open
// entry keeps fp64 sums that pass up to its parent when it completes, so the
// row data is added once.
#include "args.hpp"
#include "common.hpp"

namespace sa {

constexpr int kPyrWaves = 4;      // waves per workgroup, each with its own run of spans
constexpr int kPyrRows = 16;      // level-0 rows whose loads are in flight together
constexpr int kPyrWaveRows = 256; // level-0 rows per wave (whole spans, at least one)

// The E consecutive elements of one row that a lane owns, widened to fp32.
// Loads go through a buffer resource over the wave's run of rows: a lane's
// offset is fixed and each row's offset is a scalar, so a load takes no
// vector address arithmetic (non-temporal: the rows are read once).
constexpr int kBufNT = 2;
template <typename T, int E> struct LaneRow;
template <> struct LaneRow<bf16_t, 2> {
  uint32_t w;
  __device__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff) { w = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kBufNT); }
  __device__ float at(int j) const { return j ? bf16_hi(w) : bf16_lo(w); }
};
template <> struct LaneRow<bf16_t, 1> {
  uint16_t w;
  __device__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff) { w = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kBufNT); }
  __device__ float at(int) const { return bf16_to_f32(w); }
};
template <> struct LaneRow<float, 2> {
  vl_u32x2 w;
  __device__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff) { w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kBufNT); }
  __device__ float at(int j) const { return __uint_as_float(w[j]); }
};
template <> struct LaneRow<float, 1> {
  uint32_t w;
  __device__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff) { w = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kBufNT); }
  __device__ float at(int) const { return __uint_as_float(w); }
};

// A raw buffer resource (no stride, no format) over nbytes starting at p.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t run_rsrc(const void* p, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, nbytes, 0x00020000);
}

// Store the E means x[j] * inv, each rounded once to the element type.
template <typename T, int E>
__device__ __forceinline__ void store_means(void* p, int64_t i, const double* x, double inv) {
  if constexpr (sizeof(T) == 2 && E == 2) {
    const uint32_t w = uint32_t(f64_to_bf16(x[0] * inv)) | (uint32_t(f64_to_bf16(x[1] * inv)) << 16);
    reinterpret_cast<uint32_t*>(p)[i >> 1] = w;
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) Elem<T>::store_d(p, i + j, x[j] * inv);
  }
}

// Sums over the 64 lanes of 16 values at once. Each step halves the number of
// values a lane holds: the lane pairs that differ in one index bit (5, 4, 3,
// then 2) exchange, and each lane keeps the sum for the value that its own
// bit selects. Lane-swaps across the wave halves and across 16-lane rows, a
// half-row rotation, then a mirror within each 8 lanes; two quad exchanges
// finish the sum. Value u's total ends in lanes 4u .. 4u+3.
__device__ __forceinline__ float sum16_over_wave(const float (&v)[16], int lane) {
  float w[8], x[4], y[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]),
                                                    false, false);
    w[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);   // value i + 8 b5
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[i]), __float_as_uint(w[i + 4]),
                                                    false, false);
    x[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);   // value i + 4 b4 + 8 b5
  }
  const bool b3 = lane & 8, b2 = lane & 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float mine = b3 ? x[i + 2] : x[i], other = b3 ? x[i] : x[i + 2];
    y[i] = mine + dpp_move<0x128, 0xF>(other);              // row_ror:8 -> lane l ^ 8
  }
  const float mine = b2 ? y[1] : y[0], other = b2 ? y[0] : y[1];
  float z = mine + dpp_move<0x141, 0xF>(other);             // row_half_mirror -> lane l ^ 7
  z += dpp_move<0xB1, 0xF>(z);                              // quad_perm [1,0,3,2]
  z += dpp_move<0x4E, 0xF>(z);                              // quad_perm [2,3,0,1]
  return z;
}

template <typename T, int D, int LMAX>
__global__ __launch_bounds__(kPyrWaves * 64) void pyramid_kernel(PyramidArgs a, int spans_per_wave) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kPyrWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.y;
  const int P = a.top_span;
  const int64_t rbeg = (int64_t)wave * spans_per_wave * P;
  if (rbeg >= a.N) return;
  const int64_t rend = min<int64_t>(rbeg + (int64_t)spans_per_wave * P, a.N);
  const int64_t base = (int64_t)bh * a.N;
  float* sc = a.scores + (int64_t)bh * a.Nt;
  const int64_t col = (int64_t)E * lane;

  // open entry of each level: the fp64 sums of its q, k, v, its score so
  // far, children still to come, and its index in the level
  double acc[LMAX][3][E];
  float mx[LMAX];
  int left[LMAX];
  int64_t jnext[LMAX];
  double inv[LMAX];
  {
    int64_t w = 1;
#pragma unroll
    for (int l = 1; l < LMAX; ++l) {
      w *= a.factor;
      left[l] = a.factor;
      jnext[l] = rbeg / w;
      inv[l] = 1.0 / (double)w;
      mx[l] = -INFINITY;
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int j = 0; j < E; ++j) acc[l][t][j] = 0.0;
    }
  }
  // the next batch's loads are issued before the current batch is used
  constexpr int kRowBytes = D * Elem<T>::bytes;
  const int64_t first = (base + rbeg) * D;
  const int nbytes = (int)(rend - rbeg) * kRowBytes;
  const auto rq = run_rsrc(static_cast<const char*>(a.q) + first * Elem<T>::bytes, nbytes);
  const auto rk = run_rsrc(static_cast<const char*>(a.k) + first * Elem<T>::bytes, nbytes);
  const auto rv = run_rsrc(static_cast<const char*>(a.v) + first * Elem<T>::bytes, nbytes);
  const int voff = lane * E * Elem<T>::bytes;
  // two batches alternate: the next batch's loads are in flight while the
  // current one is used. A row's offset is wave-uniform (a scalar operand);
  // rows past the run re-read its last row, so every address stays inside it.
  struct Batch { LaneRow<T, E> q[kPyrRows], k[kPyrRows], v[kPyrRows]; };
  auto issue = [&](Batch& x, int64_t rb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kPyrRows; ++u) {
      const int soff = (int)(min(rb + u, rend - 1) - rbeg) * kRowBytes;
      x.q[u].load(rq, voff, soff);
      x.k[u].load(rk, voff, soff);
      x.v[u].load(rv, voff, soff);
    }
  };
  auto consume = [&](const Batch& x, int64_t rb) __attribute__((always_inline)) {
    float part[kPyrRows];
#pragma unroll
    for (int u = 0; u < kPyrRows; ++u) {
      float t = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) t = __builtin_fmaf(x.q[u].at(j), x.q[u].at(j), __builtin_fmaf(x.k[u].at(j), x.k[u].at(j), t));
      part[u] = t;
    }
    const float tot = sum16_over_wave(part, lane);            // row rb + lane/4
    const int nrows = (int)min<int64_t>(kPyrRows, rend - rb);
    if ((lane & 3) == 0 && (lane >> 2) < nrows) sc[rb + (lane >> 2)] = tot;
#pragma unroll
    for (int u = 0; u < kPyrRows; ++u) {
      if (LMAX > 1 && a.levels > 1 && u < nrows) {
        const float su = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tot), 4 * u));
#pragma unroll
        for (int j = 0; j < E; ++j) {
          acc[1][0][j] += (double)x.q[u].at(j);
          acc[1][1][j] += (double)x.k[u].at(j);
          acc[1][2][j] += (double)x.v[u].at(j);
        }
        mx[1] = fmaxf(mx[1], su);
        // an entry completes when its last child does; its sums and score
        // pass up to the parent's open entry
        bool carry = true;
#pragma unroll
        for (int l = 1; l < LMAX; ++l) {
          carry = carry && l < a.levels && --left[l] == 0;
          if (carry) {
            const int64_t row = (int64_t)bh * a.Nc + a.coff[l] + jnext[l];
            store_means<T, E>(a.pq, row * D + col, acc[l][0], inv[l]);
            store_means<T, E>(a.pk, row * D + col, acc[l][1], inv[l]);
            store_means<T, E>(a.pv, row * D + col, acc[l][2], inv[l]);
            if (lane == 0) sc[a.soff[l] + jnext[l]] = mx[l];
            if (l + 1 < LMAX) {
#pragma unroll
              for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int j = 0; j < E; ++j) acc[l + 1][t][j] += acc[l][t][j];
              mx[l + 1] = fmaxf(mx[l + 1], mx[l]);
            }
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
              for (int j = 0; j < E; ++j) acc[l][t][j] = 0.0;
            mx[l] = -INFINITY;
            left[l] = a.factor;
            ++jnext[l];
          }
        }
      }
    }
  };
  Batch b0, b1;
  issue(b0, rbeg);
  for (int64_t rb = rbeg; rb < rend; rb += 2 * kPyrRows) {
    issue(b1, rb + kPyrRows);
    consume(b0, rb);
    if (rb + kPyrRows >= rend) break;
    issue(b0, rb + 2 * kPyrRows);
    consume(b1, rb + kPyrRows);
  }
}

hipError_t launch_pyramid(const PyramidArgs& a, int dtype, int d, hipStream_t s) {
  if (a.top_span > 256 || a.levels > 8 || a.levels < 1 || a.N % a.top_span) return hipErrorInvalidValue;
  const int spw = max(1, kPyrWaveRows / a.top_span);
  const int nspan = a.N / a.top_span;
  const int waves = (nspan + spw - 1) / spw;
  dim3 grid((waves + kPyrWaves - 1) / kPyrWaves, a.B * a.H), block(kPyrWaves * 64);
#define SA_PYR(T_, D_)                                                                   \
  do {                                                                                   \
    if (a.levels <= 3) hipLaunchKernelGGL((pyramid_kernel<T_, D_, 3>), grid, block, 0, s, a, spw); \
    else hipLaunchKernelGGL((pyramid_kernel<T_, D_, 8>), grid, block, 0, s, a, spw);    \
  } while (0)
  if (dtype == 0 && d == 128) SA_PYR(bf16_t, 128);
  else if (dtype == 0 && d == 64) SA_PYR(bf16_t, 64);
  else if (dtype == 1 && d == 128) SA_PYR(float, 128);
  else if (dtype == 1 && d == 64) SA_PYR(float, 64);
  else return hipErrorInvalidValue;
#undef SA_PYR
  return hipGetLastError();
}

}  // namespace sa
