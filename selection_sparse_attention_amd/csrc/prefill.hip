// Chunked prefill attention over pyramid-selected entries (Lighthouse
// summary, Methodology 2C: the chosen entries form a causally consistent
// subsequence, ordinary softmax attention runs on it, and each query's output
// goes back to its own position).
//
// For query block beta of one (sequence, head), query i = 128 beta + u sees
// the block's selected entries (rows of K/V for level 0, of the coarse K/V
// levels above) and the block's own level-0 keys 128 beta .. i:
//   out[i] = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j      (fp32)
//
// gfx950 design, one 256-thread workgroup per (block, head), wave w owning
// queries 32w .. 32w+31:
//   * keys are processed in tiles of 32; the 256 threads gather a tile's K
//     and V rows by index straight from HBM into LDS (double-buffered, the
//     next tile's loads in flight during the current tile's math).  K is kept
//     row-major (rows padded to 272 B), V transposed (d rows of 32 keys,
//     padded to 72 B) - the operand layouts the matrix cores want.
//   * scores come out transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16 with
//     the query block's fragments resident in registers), so every lane holds
//     8 keys x 2 queries; a query's running max is a reduction over 8 values
//     and 4 lanes.
//   * those probabilities are already the B operand of O^T = V^T P^T, so the
//     second product needs no data movement; P is split into a bf16 high part
//     and a bf16 remainder (two products) so the weights keep ~16 bits.
//   * blocks of a head run on one die: block ids are mapped so that each of
//     the 8 dies (round-robin dispatch) serves two heads, heaviest blocks
//     first, keeping the heads' selected rows hot in that die's L2.
#include "args.hpp"
#include "common.hpp"

namespace sa {

typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));
typedef float f32x4p __attribute__((ext_vector_type(4)));

constexpr int kPfThreads = 256;
constexpr int kKT = 32;                 // keys per tile
constexpr int kD = 128;                 // head dim
constexpr int kKRow = kD + 8;           // K tile row stride (bf16 elements) = 272 B
constexpr int kVRow = 36;               // V^T tile row stride (bf16 elements) = 72 B

typedef float f32x2p __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2p __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair (round to nearest even, one instruction
// on gfx950), and the fp32 value of each half.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2p){x, y}, bf16x2p));
}

__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kD * kVRow];

  // ---- which (head, block): die-major, two heads per die, heavy first
  const int nh = a.B * a.H;
  const int hpx = (nh + 7) / 8;
  const int L = blockIdx.x;
  const int xcd = L % 8, slot = L / 8;
  const int bh = xcd + 8 * (slot % hpx);
  const int blk = a.nblk - 1 - slot / hpx;
  if (bh >= nh || blk < 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, jg = lane >> 4;
  const int q0 = blk * a.q_block;
  const int nq = min(a.q_block, a.N - q0);
  const int c_sel = min(max(a.blk_count[(int64_t)bh * a.nblk + blk], 0), a.K);
  const int32_t* list = a.blk_idx + ((int64_t)bh * a.nblk + blk) * a.K;
  const int T = c_sel + nq;
  const int ntiles = (T + kKT - 1) / kKT;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)bh * a.N * kD;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k) + (int64_t)bh * a.N * kD;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v) + (int64_t)bh * a.N * kD;
  const uint16_t* pkb = reinterpret_cast<const uint16_t*>(a.pk) + (int64_t)bh * a.Nc * kD;
  const uint16_t* pvb = reinterpret_cast<const uint16_t*>(a.pv) + (int64_t)bh * a.Nc * kD;

  // ---- query fragments (B operand of S^T = K Q^T): query 32w + 16nt + l16,
  //      dims 32 jg + 8 s .. +8
  bf16x8p qf[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int ql = 32 * wid + 16 * nt + l16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (ql < nq) w = *reinterpret_cast<const uint4*>(qb + (int64_t)(q0 + ql) * kD + 32 * jg + 8 * s);
      qf[nt][s] = __builtin_bit_cast(bf16x8p, w);
    }
  }

  // ---- gather roles: K (thread -> key t/8, 16 dims at 16*(t%8)),
  //      V (thread -> keys 2(t%16), 2(t%16)+1, 8 dims at 8*(t/16)).
  //      Entry e of the block's key sequence is selected entry e (a flat id)
  //      for e < c_sel, the block's own level-0 key q0 + e - c_sel below T,
  //      and nothing (a zero row) past T.  A flat id outside the pyramid is
  //      malformed and also reads as a zero row.
  const int gk_key = tid >> 3, gk_seg = tid & 7;
  const int gv_kp = tid & 15, gv_seg = tid >> 4;
  auto entry_id = [&](int e) -> int {
    if (e < c_sel) return list[e];
    if (e < T) return q0 + e - c_sel;
    return -1;
  };
  auto row_ptr = [&](int f, bool is_v) -> const uint16_t* {
    if ((unsigned)f >= (unsigned)(a.N + a.Nc)) return nullptr;
    if (f < a.N) return (is_v ? vb : kb) + (int64_t)f * kD;
    return (is_v ? pvb : pkb) + (int64_t)(f - a.N) * kD;
  };
  // ids run two tiles ahead of the rows, rows one tile ahead of the math
  int id_c[3], id_n[3];
  auto load_ids = [&](int tile, int* id) {
    const int e0 = tile * kKT;
    id[0] = entry_id(e0 + gk_key);
    id[1] = entry_id(e0 + 2 * gv_kp);
    id[2] = entry_id(e0 + 2 * gv_kp + 1);
  };
  uint4 rk[2], rv[2];
  auto gather = [&](const int* id) {
    const uint16_t* pk = row_ptr(id[0], false);
    if (pk) {
      rk[0] = *reinterpret_cast<const uint4*>(pk + 16 * gk_seg);
      rk[1] = *reinterpret_cast<const uint4*>(pk + 16 * gk_seg + 8);
    } else {
      rk[0] = rk[1] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint16_t* pv = row_ptr(id[1 + r], true);
      rv[r] = pv ? *reinterpret_cast<const uint4*>(pv + 8 * gv_seg) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
    uint16_t* kdst = s_k[buf] + gk_key * kKRow + 16 * gk_seg;
    *reinterpret_cast<uint4*>(kdst) = rk[0];
    *reinterpret_cast<uint4*>(kdst + 8) = rk[1];
    // V^T: dims 8 gv_seg + i, keys 2 gv_kp and 2 gv_kp + 1 packed in one dword
    const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&rv[0]);
    const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&rv[1]);
    uint16_t* vdst = s_vt[buf] + (8 * gv_seg) * kVRow + 2 * gv_kp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a0 = v0[i], a1 = v1[i];
      *reinterpret_cast<uint32_t*>(vdst + (2 * i) * kVRow) = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
      *reinterpret_cast<uint32_t*>(vdst + (2 * i + 1) * kVRow) = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    }
  };

  // ---- running state for queries 32w + 16nt + l16
  float m[2] = {-INFINITY, -INFINITY}, lpart[2] = {0.f, 0.f};
  f32x4p o[8][2];                                   // O^T[d = 16 dt + 4 jg + i][q]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o[dt][nt] = (f32x4p){0.f, 0.f, 0.f, 0.f};
  const float sc = a.scale_log2;

  if (ntiles > 0) {
    load_ids(0, id_c);
    gather(id_c);
    if (ntiles > 1) load_ids(1, id_c);
    stash(0);
  }
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 2 < ntiles) load_ids(tile + 2, id_n);
    if (tile + 1 < ntiles) gather(id_c);
    const uint16_t* kt = s_k[buf];
    const uint16_t* vt = s_vt[buf];
    // S^T[key = 16 mt + 4 jg + i][q = 16 nt + l16]
    f32x4p s[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      bf16x8p kf[4];
#pragma unroll
      for (int st = 0; st < 4; ++st)
        kf[st] = __builtin_bit_cast(bf16x8p,
                                    *reinterpret_cast<const uint4*>(kt + (16 * mt + l16) * kKRow + 32 * jg + 8 * st));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4p c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st], qf[nt][st], c, 0, 0, 0);
        s[mt][nt] = c;
      }
    }
    // scale (log2 domain), mask only on tiles that reach past the selection
    const int e0 = tile * kKT;
    float x[2][2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[nt][mt][i] = s[mt][nt][i] * sc;
    if (e0 + kKT > c_sel) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int ql = 32 * wid + 16 * nt + l16;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = e0 + 16 * mt + 4 * jg + i;
            const bool ok = (e < c_sel) || (e < T && (e - c_sel) <= ql);
            if (!ok) x[nt][mt][i] = -INFINITY;
          }
      }
    }
    // online softmax per query; P^T fragments as a bf16 high part and a bf16
    // remainder (the weights keep ~16 bits through the second product)
    uint4 ph[2], pl[2];
    float alpha[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float tmax = x[nt][0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, x[nt][mt][i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mn = fmaxf(m[nt], tmax);
      const float msub = (mn == -INFINITY) ? 0.f : mn;   // a fully masked row stays at p = 0
      alpha[nt] = __builtin_amdgcn_exp2f(m[nt] - msub);
      m[nt] = mn;
      float p[8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[4 * mt + i] = __builtin_amdgcn_exp2f(x[nt][mt][i] - msub);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ps += p[j];
      lpart[nt] = lpart[nt] * alpha[nt] + ps;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t h = pk_bf16(p[2 * j], p[2 * j + 1]);
        const float r0 = p[2 * j] - __builtin_bit_cast(float, h << 16);
        const float r1 = p[2 * j + 1] - __builtin_bit_cast(float, h & 0xFFFF0000u);
        hw[j] = h;
        lw[j] = pk_bf16(r0, r1);
      }
      ph[nt] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      pl[nt] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    // rescale the accumulators only when some query's running max moved
    if (!__all(alpha[0] == 1.f && alpha[1] == 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[dt][nt] *= alpha[nt];
    }
    // O^T += V^T P^T over the tile's 32 keys: k-slot j of lane group jg is
    // key 4 jg + j (j < 4) or 16 + 4 jg + (j - 4)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* vrow = vt + (16 * dt + l16) * kVRow;
      const uint2 w0 = *reinterpret_cast<const uint2*>(vrow + 4 * jg);
      const uint2 w1 = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * jg);
      const bf16x8p vf = __builtin_bit_cast(bf16x8p, make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8p, ph[nt]), o[dt][nt], 0, 0, 0);
        o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8p, pl[nt]), o[dt][nt], 0, 0, 0);
      }
    }
    if (tile + 1 < ntiles) {
      stash(buf ^ 1);
#pragma unroll
      for (int j = 0; j < 3; ++j) id_c[j] = id_n[j];
    }
    __syncthreads();
  }

  // ---- normalise and write: lane holds d = 16 dt + 4 jg + 0..3 of query
  //      32w + 16 nt + l16
  float* ob = a.out + (int64_t)bh * a.N * kD;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float lt = lpart[nt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int ql = 32 * wid + 16 * nt + l16;
    if (ql < nq) {
      const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
      float* orow = ob + (int64_t)(q0 + ql) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4p v = o[dt][nt] * inv;
        *reinterpret_cast<float4*>(orow + 16 * dt + 4 * jg) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, int d, hipStream_t s) {
  if (d != kD || a.q_block != 128) return hipErrorInvalidValue;
  const int nh = a.B * a.H;
  const int hpx = (nh + 7) / 8;
  dim3 grid(8 * hpx * a.nblk);
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(kPfThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
