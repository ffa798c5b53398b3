// Low-rank pre-RoPE token index ("Full Attention Strikes Back" summary,
// Methodology item 2): a 16-dim projector is applied to the query and key
// features before RoPE, and relevance is later estimated in that subspace.
//
// k_idx[b,g,j,c] = sum_e P_k[g,c,e] * k_pre[b,g,j,e]   (fp32, rounded once)
// q_idx[b,h,c]   = sum_e P_q[g,c,e] * q_pre[b,h,e]     (fp32)
//
// Key side: an HBM-bound stream over k_pre (d * e bytes in, 16 * e out per
// token).  bf16 rows go through the matrix cores (project_rows_mfma below:
// 16-row tiles, the fp32 projector split into three bf16 parts).  fp32 rows
// take a vector path: L = d / (16 bytes / e) lanes share a token: each loads 16
// contiguous bytes of its row (so one wave instruction reads 64 / L whole
// rows) and multiplies them with its slice of the projector, which it holds
// in registers for the whole launch (16 outputs x 16 bytes of dims).  A
// recursive-halving exchange across the token's lanes then sums the 16
// partial outputs, leaving output c on lane c of the token (outputs 2c and
// 2c + 1 on lane c when L = 8; output c on lanes 2c and 2c + 1 when L = 32),
// so a token's 16 outputs are stored contiguously.  Every token goes
// through the same order of operations, so appending rows one at a time
// gives the same bits as a full build.  Query side: the last workgroup of each
// (sequence, group) projects the group's query heads the same way (they are
// consecutive rows of q_pre).
#include "args.hpp"
#include "common.hpp"
#include "index_project.hpp"

namespace sa {

constexpr int kIdxThreads = 256;

template <typename T, int D>
struct IdxGeom {
  static constexpr int E = 16 / (int)sizeof(T);    // dims per lane (one 16-byte load)
  static constexpr int L = D / E;                  // lanes per token
  static constexpr int TPW = 64 / L;               // tokens per wave step
};

// One 16-byte slice of a key row, widened to fp32.
template <typename T> struct Slice;
template <> struct Slice<bf16_t> {
  static constexpr int E = 8;
  vl_u32x4 w;
  __device__ void load(const void* base, int64_t elem) {
    w = __builtin_nontemporal_load(reinterpret_cast<const vl_u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem));
  }
  __device__ float get(int i) const { return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]); }
};
template <> struct Slice<float> {
  static constexpr int E = 4;
  vl_f32x4 w;
  __device__ void load(const void* base, int64_t elem) {
    w = __builtin_nontemporal_load(reinterpret_cast<const vl_f32x4*>(reinterpret_cast<const float*>(base) + elem));
  }
  __device__ float get(int i) const { return w[i]; }
};

// Sum the 16 per-lane partial outputs over the L lanes of a token (lanes
// l0 .. l0 + L - 1, l0 a multiple of L): recursive halving, each step keeps
// the half of the outputs selected by one bit of the lane index.  Returns
// with acc[0 .. 16/L) holding outputs  (lane % L) * (16/L) + i; for L = 32
// the last step adds two lanes that hold the same output, so lanes 2c and
// 2c + 1 of a token both end with output c.
// A value from lane (lane ^ S).  Inside a 16-lane row by DPP (VALU moves):
// quad permutes for S = 1, 2; a rotate by 8 for S = 8; for S = 4 the lanes
// with bit 2 set take the rotate by 4 (from lane - 4) and the others the
// rotate by 12 (from lane + 4).  S = 16 and 32 go through ds_bpermute.
template <int CTRL>
__device__ __forceinline__ float dpp_xf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int S>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  if constexpr (S == 1) return dpp_xf<0xB1>(v);         // quad_perm [1,0,3,2]
  else if constexpr (S == 2) return dpp_xf<0x4E>(v);    // quad_perm [2,3,0,1]
  else if constexpr (S == 4) {
    const float from_below = dpp_xf<0x124>(v), from_above = dpp_xf<0x12C>(v);   // row_ror 4 / 12
    return (lane & 4) ? from_below : from_above;
  } else if constexpr (S == 8) return dpp_xf<0x128>(v);  // row_ror 8
  else return __shfl_xor(v, S);
}

// One halving step over lane bit S with N outputs still held (compile-time
// sizes, so every register index is static).
template <int S, int N>
__device__ __forceinline__ void rs_step(float (&acc)[16], int lane) {
  if constexpr (S >= 1) {
    if constexpr (N > 1) {
      constexpr int H = N / 2;
      // lanes with bit S set keep the upper half (and send the lower)
      const bool upper = (lane & S) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float keep = upper ? acc[H + i] : acc[i];
        const float give = upper ? acc[i] : acc[H + i];
        acc[i] = keep + xor_lane<S>(give, lane);
      }
      rs_step<S / 2, H>(acc, lane);
    } else {
      acc[0] += xor_lane<S>(acc[0], lane);
      rs_step<S / 2, 1>(acc, lane);
    }
  }
}

template <int L>
__device__ __forceinline__ void reduce_scatter16(float (&acc)[16]) {
  rs_step<L / 2, 16>(acc, threadIdx.x & 63);
}

// Project rows [first, last) of src (row r at element (row0 + r) * D) with
// the projector P (16 x D fp32): dst[(row0 + r) * 16 + c], in the element
// type of OutT.  The workgroup's waves take TPW rows per step each, U steps
// of loads in flight (16 for builds: with two waves per SIMD the stream needs
// that many rows in flight; 1 for appends, where only latency counts).
template <typename T, int D, typename OutT, int U>
__device__ __forceinline__ void project_rows(const void* src, const float* Pg, void* dst, int64_t row0,
                                             int first, int last) {
  using GM = IdxGeom<T, D>;
  constexpr int E = GM::E, L = GM::L, TPW = GM::TPW;
  constexpr int OUTS = (16 / L) > 0 ? (16 / L) : 1;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // this lane's slice of the projector: dims e0 .. e0 + E of every output
  const int sl = lane % L;
  const int e0 = sl * E;
  float P[16][E];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
#pragma unroll
    for (int q = 0; q < E; q += 4) {
      const vl_f32x4 v = *reinterpret_cast<const vl_f32x4*>(Pg + c * D + e0 + q);
      P[c][q] = v[0]; P[c][q + 1] = v[1]; P[c][q + 2] = v[2]; P[c][q + 3] = v[3];
    }
  }
  const int tw = lane / L;                         // this lane's row within a wave step
  constexpr int STEP = TPW * (kIdxThreads / 64);   // rows per workgroup step
  for (int base = first; base < last; base += STEP * U) {
    Slice<T> s[U];
    int row[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      row[u] = base + (u * (kIdxThreads / 64) + wid) * TPW + tw;
      s[u].load(src, (row0 + min(row[u], last - 1)) * D + e0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        float x = 0.f;
#pragma unroll
        for (int q = 0; q < E; ++q) x = fmaf(P[c][q], s[u].get(q), x);
        acc[c] = x;
      }
      reduce_scatter16<L>(acc);
      if (row[u] < last) {
        if (L <= 16) {
#pragma unroll
          for (int i = 0; i < OUTS; ++i) Elem<OutT>::store(dst, (row0 + row[u]) * 16 + sl * OUTS + i, acc[i]);
        } else if ((sl & 1) == 0) {
          Elem<OutT>::store(dst, (row0 + row[u]) * 16 + (sl >> 1), acc[0]);
        }
      }
    }
  }
}

// The projection of rows [first, last) of src (row r at element (row0 + r) *
// D) into dst[(row0 + r) * 16 + c], in the element type of OutT.
template <int D, typename OutT, int U>
__device__ __forceinline__ void project_rows_mfma(const void* src, const float* Pg, void* dst, int64_t row0,
                                                  int first, int last) {
  project_rows_mfma_st<D, U, kIdxThreads>(src, Pg, row0, first, last,
                                          [&](int r, int col, float v) __attribute__((always_inline)) {
                                            Elem<OutT>::store(dst, (row0 + r) * 16 + col, v);
                                          });
}

template <typename T, int D, int U>
__global__ __launch_bounds__(kIdxThreads) void index_lowrank_kernel(IndexLowrankArgs a) {
  const int gi = blockIdx.y, b = blockIdx.z;
  const int g = a.groups.ids[gi];
  const int n_tok = a.t1 - a.t0;
  const int per_wg = (int)a.tokens_per_wg;
  const int kblocks = (n_tok + per_wg - 1) / per_wg;
  constexpr bool kMfma = sizeof(T) == 2;
  if ((int)blockIdx.x == kblocks) {
    // query side: the group's G query heads are G consecutive rows of q_pre
    if (a.q_pre == nullptr) return;
    if constexpr (kMfma)
      project_rows_mfma<D, float, 1>(a.q_pre, a.proj_q + (int64_t)g * 16 * D, a.q_idx,
                                     (int64_t)b * a.Hq + (int64_t)g * a.G, 0, a.G);
    else
      project_rows<T, D, float, 1>(a.q_pre, a.proj_q + (int64_t)g * 16 * D, a.q_idx,
                                   (int64_t)b * a.Hq + (int64_t)g * a.G, 0, a.G);
    return;
  }
  const int first = a.t0 + (int)blockIdx.x * per_wg;
  if constexpr (kMfma)
    project_rows_mfma<D, T, U>(a.k_pre, a.proj_k + (int64_t)g * 16 * D, a.k_idx,
                                            ((int64_t)b * a.Hkv + g) * a.n_cap, first,
                                            min(first + per_wg, a.t1));
  else
    project_rows<T, D, T, U>(a.k_pre, a.proj_k + (int64_t)g * 16 * D, a.k_idx,
                             ((int64_t)b * a.Hkv + g) * a.n_cap, first, min(first + per_wg, a.t1));
}

hipError_t launch_index_lowrank(const IndexLowrankArgs& a, int dtype, int d, hipStream_t s) {
  const int n_tok = a.t1 - a.t0;
  const int kblocks = (n_tok + a.tokens_per_wg - 1) / a.tokens_per_wg;
  dim3 grid(kblocks + 1, a.groups.n, a.B), block(kIdxThreads);
  const bool build = n_tok > 64;
#define SA_IDX(T_, D_)                                                                       \
  do {                                                                                       \
    if (build) hipLaunchKernelGGL((index_lowrank_kernel<T_, D_, 8>), grid, block, 0, s, a); \
    else hipLaunchKernelGGL((index_lowrank_kernel<T_, D_, 1>), grid, block, 0, s, a);        \
  } while (0)
  if (dtype == 0 && d == 128) SA_IDX(bf16_t, 128);
  else if (dtype == 0 && d == 64) SA_IDX(bf16_t, 64);
  else if (dtype == 1 && d == 128) SA_IDX(float, 128);
  else if (dtype == 1 && d == 64) SA_IDX(float, 64);
  else return hipErrorInvalidValue;
#undef SA_IDX
  return hipGetLastError();
}

}  // namespace sa
