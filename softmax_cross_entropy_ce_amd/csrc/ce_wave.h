// Path 5: rows of up to 16 KB held whole in one wavefront's registers.
//
// Rows of a few hundred to a few thousand elements are too long for the
// many-rows-per-wave layout of path 1 and too short for a workgroup per
// row: a persistent workgroup with one row in flight leaves most of a
// compute unit's memory pipeline idle.  Here each 64-lane wave takes R
// consecutive rows and issues the loads of all of them at once; lane q
// holds vectors q, q+64, ..., q+64(NV-1) of each row, VB bytes (VW
// elements) per vector, LB = NV * VB bytes of a row per lane.  The row's
// max, its sum of exponentials without the target and its outputs follow
// from registers, with the wave-wide DPP reductions of ce_device.h: no
// LDS, no barrier, no second read.  Workgroups of four waves are not
// persistent; the grid covers the rows once.
//
// The host picks VB as the widest of 16, 8 and 4 bytes that every row
// start of every array is aligned to and that divides every row length and
// stride, so a vector lies wholly inside or wholly outside its row; lanes
// past the row's end read zeros through the buffer resource's bound (and
// are masked out of the reductions) and their stores are dropped by it.
//
// The arithmetic is that of the other row kernels (ce_rowops.h): with
// cg = round(max z * log2 e), every term is 2^(z log2e - cg) formed with
// one fma, the target's term is left out of the sum, and the sum adds each
// vector's terms as a pairwise tree, then the vectors in slot order, then
// the lanes with the fixed DPP tree, so the bits do not depend on timing.
// For float32 the terms of the sum replace z in the registers and the
// gradient is one multiply per element; 16-bit rows recompute the terms
// (a float copy would double their registers).
#pragma once

#include "ce_rowops.h"

namespace ce {

constexpr int kWaveThreads = 256;   // four waves, each its own rows

// Raw VB-byte vectors: one buffer load each, split into 32-bit words.
template <int VB>
struct RawVec;
template <>
struct RawVec<4> {
  using W = unsigned;
  static constexpr int kWords = 1;
  __device__ static __forceinline__ W load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicyStream);
  }
  __device__ static __forceinline__ unsigned word(W w, int) { return w; }
  __device__ static __forceinline__ W from_words(const unsigned (&d)[1]) { return d[0]; }
};
template <>
struct RawVec<8> {
  using W = u32x2;
  static constexpr int kWords = 2;
  __device__ static __forceinline__ W load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyStream);
  }
  __device__ static __forceinline__ unsigned word(W w, int k) { return k == 0 ? w.x : w.y; }
  __device__ static __forceinline__ W from_words(const unsigned (&d)[2]) { return W{d[0], d[1]}; }
};
template <>
struct RawVec<16> {
  using W = u32x4;
  static constexpr int kWords = 4;
  __device__ static __forceinline__ W load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyStream);
  }
  __device__ static __forceinline__ unsigned word(W w, int k) {
    return k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
  }
  __device__ static __forceinline__ W from_words(const unsigned (&d)[4]) {
    return W{d[0], d[1], d[2], d[3]};
  }
};

template <typename T, int VB>
__device__ __forceinline__ void widen_vec(typename RawVec<VB>::W w, float (&f)[VB / sizeof(T)]) {
  constexpr int PER = 4 / (int)sizeof(T);  // elements per word
#pragma unroll
  for (int i = 0; i < VB / (int)sizeof(T); ++i)
    f[i] = widen_half<T>(RawVec<VB>::word(w, i / PER), i % PER);
}

// VB: vector bytes (16, 8 or 4); LB: bytes of a row per lane (16 to 256);
// R rows per wave.
template <typename T, int VB, int LB, bool GRAD, int OP>
__global__ __launch_bounds__(kWaveThreads) void ce_wave_kernel(const T* __restrict__ logits,
                                                               const int32_t* __restrict__ targets,
                                                               int64_t B, int C, RowArgs rs,
                                                               T* __restrict__ grad,
                                                               float* __restrict__ loss_rows) {
  constexpr uint32_t ES = sizeof(T);
  constexpr int VW = VB / (int)ES;          // elements per vector
  constexpr int NV = LB / VB;               // vectors of a row per lane
  constexpr int R = LB >= 128 ? 1 : 128 / LB;
  constexpr bool kKeep = GRAD && ES == 4;
  static_assert(VB == 4 || VB == 8 || VB == 16, "vector bytes");
  static_assert(NV >= 1 && LB % VB == 0, "lane bytes");
  using RV = RawVec<VB>;
  using W = typename RV::W;

  const int lane = threadIdx.x & 63;
  const int64_t row0 =
      ((int64_t)blockIdx.x * (kWaveThreads / 64) +
       __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))) * R;
  if (row0 >= B) return;  // whole wave; there is no barrier
  const float invB = row_invB(rs), gmul = grad_mul(rs);
  const int nvec = C / VW;  // vectors per row
  const uint32_t lane_off = (uint32_t)lane * VB;

  // every load of the wave's rows; rows past B get an empty resource
  W w[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = row0 + r < B;  // uniform
    const rsrc_t rin = make_rsrc(logits + (live ? row0 + r : row0) * rs.ldz,
                                 live ? (uint32_t)C * ES : 0u);
#pragma unroll
    for (int j = 0; j < NV; ++j) w[r][j] = RV::load(rin, lane_off + (uint32_t)(j * 64 * VB));
  }

  // Per-row work that does not touch the elements runs across lanes: lane
  // r < R reads row r's target (and later computes row r's epilogue), and
  // each row's target column is read from its lane.  Vector tv = t / VW of
  // a row sits in lane tv % 64, slot tv / 64.
  const bool tlive = lane < R && row0 + lane < B;
  const RowTarget rl = tlive ? row_target<OP>(targets, row0 + lane, C, rs)
                             : RowTarget{-1, false, false};
  int tc[R], tl[R], ts[R], tj[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = __builtin_amdgcn_readlane(rl.t, r);
    tc[r] = t;
    tl[r] = t >= 0 ? (t / VW) & 63 : -1;
    ts[r] = t >= 0 ? (t / VW) >> 6 : -1;
    tj[r] = t >= 0 ? t % VW : 0;
  }

  // max and target logit of each row (the target's 32-bit word is picked
  // from the raw vector, read from its lane and widened)
  constexpr int PER = 4 / (int)ES;  // elements per word
  float cg[R], zt[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float m = kNegInf;
    unsigned zw = 0u;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float f[VW];
      widen_vec<T, VB>(w[r][j], f);
      const float vm = max_of(f);
      m = j * 64 + lane < nvec ? fmax2(m, vm) : m;
      if (j == ts[r]) {  // uniform
#pragma unroll
        for (int k = 0; k < RV::kWords; ++k) zw = k == tj[r] / PER ? RV::word(w[r][j], k) : zw;
      }
    }
    cg[r] = wave_allreduce(m, OpMax{}) * kLog2e;
    zt[r] = tc[r] >= 0
                ? widen_half<T>((unsigned)__builtin_amdgcn_readlane((int)zw, tl[r]), tj[r] % PER)
                : 0.f;
  }

  // The empty asm makes each 16-bit vector opaque, so that the compiler
  // widens it again in the next pass instead of keeping the widened copy
  // of this one alive (twice the registers).
  auto opaque = [&] {
    if constexpr (ES == 2) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NV; ++j) asm volatile("" : "+v"(w[r][j]));
    }
  };
  opaque();

  // sum of the terms without the target's
  float sx[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (j * 64 >= nvec) continue;  // uniform: no lane of this slot is in the row
      float f[VW], e[VW];
      widen_vec<T, VB>(w[r][j], f);
      const bool in = j * 64 + lane < nvec;
      const bool own = j == ts[r] && lane == tl[r];
#pragma unroll
      for (int i = 0; i < VW; ++i) {
        const float x = (!in || (own && i == tj[r])) ? kNegInf : f[i];
        e[i] = exp2_hw(__builtin_fmaf(x, kLog2e, -cg[r]));
      }
      s = s + tree_sum(e);
      if constexpr (kKeep) {
        unsigned d[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) d[i] = __builtin_bit_cast(unsigned, e[i]);
        w[r][j] = RV::from_words(d);
      }
    }
    sx[r] = wave_allreduce(s, OpAdd{});
  }

  // the epilogue of row r in lane r, its per-row output stored from there
  float c_l = 0.f, s_l = 1.f, z_l = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    c_l = lane == r ? cg[r] : c_l;
    s_l = lane == r ? sx[r] : s_l;
    z_l = lane == r ? zt[r] : z_l;
  }
  const RowResult res = row_finish<OP>(c_l, s_l, z_l, rl.valid, rl.ignored, invB, gmul);
  if (tlive) store_row<OP>(loss_rows, row0 + lane, res, c_l, s_l, z_l, rl.t >= 0);
  if constexpr (!GRAD) return;
  RowResult rr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rr[r].scale = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, res.scale), r));
    rr[r].gt = __builtin_bit_cast(float,
                                  __builtin_amdgcn_readlane(__builtin_bit_cast(int, res.gt), r));
  }

  // outputs from the registers
  opaque();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = row0 + r < B;  // uniform
    const rsrc_t rout = make_rsrc(grad + (live ? row0 + r : row0) * rs.ldg,
                                  live ? (uint32_t)C * ES : 0u);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (j * 64 >= nvec) continue;  // uniform
      float g[VW];
      if constexpr (kKeep) {
        float e[VW];
        widen_vec<T, VB>(w[r][j], e);
#pragma unroll
        for (int i = 0; i < VW; ++i) g[i] = e[i] * rr[r].scale;
      } else {
        float f[VW];
        widen_vec<T, VB>(w[r][j], f);
#pragma unroll
        for (int i = 0; i < VW; ++i)
          g[i] = exp2_hw(__builtin_fmaf(f[i], kLog2e, -cg[r])) * rr[r].scale;
      }
      if (j == ts[r] && lane == tl[r]) {
#pragma unroll
        for (int i = 0; i < VW; ++i) g[i] = i == tj[r] ? rr[r].gt : g[i];
      }
      VecIO<T, VW>::store(rout, lane_off + (uint32_t)(j * 64 * VB), g);
    }
  }
}

// Softmax backward on path 5 (rumus project page, milestone M8c): per row
// dot = sum_c y_c dy_c and dx_c = y_c (dy_c - dot), with whole rows of y
// and dy in a wave's registers (R * LB = 64 bytes of each array per lane,
// rows of up to 8 KB).  The dot adds each vector's products as a pairwise
// tree, the slots' sums as a pairwise tree, then the lanes with the DPP
// tree: a fixed order whose longest chain of dependent additions is below
// 16.  Lanes past a row's end load zeros, whose products add nothing.  dx
// may be y or dy: a wave reads all of its rows before it writes any.
template <typename T, int VB, int LB>
__global__ __launch_bounds__(kWaveThreads) void sm_bwd_wave_kernel(const T* __restrict__ y,
                                                                   const T* __restrict__ dy,
                                                                   int64_t B, int C,
                                                                   T* __restrict__ dx) {
  constexpr uint32_t ES = sizeof(T);
  constexpr int VW = VB / (int)ES;
  constexpr int NV = LB / VB;
  constexpr int R = LB >= 64 ? 1 : 64 / LB;
  static_assert(VB == 4 || VB == 8 || VB == 16, "vector bytes");
  static_assert(NV >= 1 && LB % VB == 0, "lane bytes");
  using RV = RawVec<VB>;
  using W = typename RV::W;

  const int lane = threadIdx.x & 63;
  const int64_t row0 =
      ((int64_t)blockIdx.x * (kWaveThreads / 64) +
       __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))) * R;
  if (row0 >= B) return;  // whole wave; there is no barrier
  const int nvec = C / VW;
  const uint32_t lane_off = (uint32_t)lane * VB;

  W wy[R][NV], wd[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = row0 + r < B;  // uniform
    const int64_t off = (live ? row0 + r : row0) * (int64_t)C;
    const uint32_t bytes = live ? (uint32_t)C * ES : 0u;
    const rsrc_t ry = make_rsrc(y + off, bytes), rd = make_rsrc(dy + off, bytes);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      wy[r][j] = RV::load(ry, lane_off + (uint32_t)(j * 64 * VB));
      wd[r][j] = RV::load(rd, lane_off + (uint32_t)(j * 64 * VB));
    }
  }

  float dot[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float part[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float a[VW], b[VW], p[VW];
      widen_vec<T, VB>(wy[r][j], a);
      widen_vec<T, VB>(wd[r][j], b);
#pragma unroll
      for (int i = 0; i < VW; ++i) p[i] = a[i] * b[i];
      part[j] = tree_sum(p);
    }
    dot[r] = wave_allreduce(tree_sum(part), OpAdd{});
  }

  // 16-bit vectors are widened again below rather than kept widened
  if constexpr (ES == 2) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        asm volatile("" : "+v"(wy[r][j]));
        asm volatile("" : "+v"(wd[r][j]));
      }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = row0 + r < B;  // uniform
    const rsrc_t ro = make_rsrc(dx + (live ? row0 + r : row0) * (int64_t)C,
                                live ? (uint32_t)C * ES : 0u);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (j * 64 >= nvec) continue;  // uniform
      float a[VW], b[VW], g[VW];
      widen_vec<T, VB>(wy[r][j], a);
      widen_vec<T, VB>(wd[r][j], b);
#pragma unroll
      for (int i = 0; i < VW; ++i) g[i] = a[i] * (b[i] - dot[r]);
      VecIO<T, VW>::store(ro, lane_off + (uint32_t)(j * 64 * VB), g);
    }
  }
}

}  // namespace ce
