// Backward of the row-wise softmax (rumus project page, milestone M8c:
// softmax forward and backward kernels).  From the forward's output y and
// the upstream gradient dy, per row:
//   dot  = sum_c y_c dy_c
//   dx_c = y_c (dy_c - dot)
// the vector-Jacobian product of y = softmax(x), since dy_j/dx_c =
// y_j ([j == c] - y_c).  Three arrays of the same type and shape, in
// float32 arithmetic; each row of y and dy is read from HBM once where the
// kernel holds it on chip, and dx is written once.
//
// Layouts, as for the loss:
//   short rows   S lanes per row inside a wave (S = 1..16), the dot reduced
//                over the segment with DPP, nothing in LDS; rows that
//                16-byte vectors do not divide go through LDS in chunks of
//                whole 16-byte vectors (the staged layout);
//   other rows   one workgroup per row at a time, persistent over rows:
//                thread i holds vectors i, i + NT, ... (NV each of y and
//                dy) in registers, the dot goes through the wave and an
//                LDS exchange in a fixed order, and the next row's loads
//                are issued while this row's dx is formed and written.
//                Vectors of a row beyond NT * NV are streamed: read for
//                the dot and read again for dx.
// The order of every sum is fixed, so results are reproducible bit for bit.
#pragma once

#include "ce_kernels.h"

namespace ce {

// ---------------------------------------------------------------------------
// Short rows: lane q of a segment holds the vectors q, q + S, ... of its row
// (VW elements each, EPL in all) of both y and dy.
// ---------------------------------------------------------------------------
template <typename T, int S, int EPL, int VW>
__global__ __launch_bounds__(kShortThreads) void sm_bwd_short_kernel(
    const T* __restrict__ y, const T* __restrict__ dy, int64_t B, int C, T* __restrict__ dx) {
  constexpr int RPB = kShortThreads / S;
  constexpr int NVEC = EPL / VW;
  static_assert(EPL % VW == 0, "EPL must be a multiple of VW");
  constexpr uint32_t ES = sizeof(T);
  const int tid = threadIdx.x;
  const int q = tid % S;
  const int64_t row0 = (int64_t)blockIdx.x * RPB;
  const int64_t nrows = (B - row0) < RPB ? (B - row0) : RPB;
  const uint32_t bytes = (uint32_t)(nrows * C * ES);
  const rsrc_t ry = make_rsrc(y + row0 * C, bytes);
  const rsrc_t rd = make_rsrc(dy + row0 * C, bytes);
  const rsrc_t ro = make_rsrc(dx + row0 * C, bytes);
  const uint32_t rowoff = (uint32_t)(tid / S) * (uint32_t)C * ES;

  float fy[EPL], fd[EPL];
#pragma unroll
  for (int j = 0; j < NVEC; ++j) {
    const int c0 = (j * S + q) * VW;
    float a[VW], b[VW];
    if (c0 < C) {
      VecIO<T, VW>::load(ry, rowoff + (uint32_t)c0 * ES, a);
      VecIO<T, VW>::load(rd, rowoff + (uint32_t)c0 * ES, b);
    } else {
#pragma unroll
      for (int w = 0; w < VW; ++w) a[w] = b[w] = 0.f;
    }
#pragma unroll
    for (int w = 0; w < VW; ++w) {
      fy[j * VW + w] = a[w];
      fd[j * VW + w] = b[w];
    }
  }
  float p[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) p[i] = fy[i] * fd[i];
  const float dot = seg_allreduce<S>(tree_sum(p), OpAdd{});
#pragma unroll
  for (int j = 0; j < NVEC; ++j) {
    const int c0 = (j * S + q) * VW;
    if (c0 < C) {
      float g[VW];
#pragma unroll
      for (int w = 0; w < VW; ++w) g[w] = fy[j * VW + w] * (fd[j * VW + w] - dot);
      VecIO<T, VW>::store(ro, rowoff + (uint32_t)c0 * ES, g);
    }
  }
}

// ---------------------------------------------------------------------------
// Rows of more than 64 bytes whose length in bytes is not a multiple of 16
// (odd lengths, ...), with y, dy and dx 16-byte aligned: the short kernel
// would read them with 8-, 4- or 2-byte loads.  As in ce_staged_kernel,
// chunks of whole passes of 256/S rows move between HBM and LDS with whole
// 16-byte loads and stores (half that kernel's chunk for each of y and
// dy), each row is reduced by a segment of S lanes reading slots q, q+S,
// ... of y and dy from LDS (read unconditionally from a stage with slack,
// their products taken as 0 past the row's end), and dx is formed in place
// of y in LDS and leaves with the chunk.  Persistent, with the loads of the
// next two chunks in flight in two register sets.
// ---------------------------------------------------------------------------
constexpr int kStagedBwdChunkBytes = kStagedChunkBytes / 2;

template <typename T, int S, int EPL>
__global__ __launch_bounds__(kStagedThreads) void sm_bwd_staged_kernel(
    const T* __restrict__ y, const T* __restrict__ dy, int64_t B, int C, T* __restrict__ dx) {
  using E = Elem<T>;
  constexpr int ES = sizeof(T), NT = kStagedThreads;
  constexpr int RPP = NT / S;
  constexpr int K = kStagedBwdChunkBytes / (16 * NT);
  constexpr int SLACK = (S * EPL * ES + 15) / 16;
  static_assert(S == 8 || S == 16 || S == 32, "segment size");
  __shared__ u32x4 sy[NT * K + SLACK], sd[NT * K + SLACK];
  const int tid = threadIdx.x, q = tid % S, seg = tid / S;
  const uint32_t voff = (uint32_t)tid * 16u;
  const int ROWS = staged_rows_per_chunk(C, ES, RPP, kStagedBwdChunkBytes);
  const int64_t nchunks = (B + ROWS - 1) / ROWS;
  const int64_t nfull = B / ROWS;
  const uint32_t full_bytes = (uint32_t)(ROWS * C * ES);
  const int nvec = (int)(full_bytes / 16);
  const int lim = C - q;  // slot k of this lane lies in the row iff k * S < lim
  int64_t chunk = blockIdx.x;
  if (chunk >= nchunks) return;  // whole workgroup

  auto load_full = [&](int64_t ch, u32x4 (&a)[K], u32x4 (&b)[K]) {
    const rsrc_t ra = make_rsrc(y + ch * ROWS * C, full_bytes);
    const rsrc_t rb = make_rsrc(dy + ch * ROWS * C, full_bytes);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      a[k] = bload128<kPolicyStream>(ra, voff, (uint32_t)k * NT * 16u);
      b[k] = bload128<kPolicyStream>(rb, voff, (uint32_t)k * NT * 16u);
    }
  };
  const int64_t G = gridDim.x;
  auto step = [&](u32x4 (&a)[K], u32x4 (&b)[K], int64_t ch) {
    const int64_t row0 = ch * ROWS;
    const bool full = ch < nfull;
    const int nrows = full ? ROWS : (int)(B - row0);
    if (full) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int gv = tid + k * NT;
        if (gv < nvec) {
          sy[gv] = a[k];
          sd[gv] = b[k];
        }
      }
    } else {
      for (int i = tid; i < nrows * C; i += NT) {
        LdsElem<T>::put(sy, i, E::load1(y + row0 * C + i));
        LdsElem<T>::put(sd, i, E::load1(dy + row0 * C + i));
      }
    }
    __syncthreads();
    if (ch + 2 * G < nfull) load_full(ch + 2 * G, a, b);

#pragma unroll 1
    for (int lr = seg; lr < nrows; lr += RPP) {  // whole segments
      const int base = lr * C + q;
      float fy[EPL], fd[EPL], p[EPL];
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        fy[k] = LdsElem<T>::get(sy, base + k * S);
        fd[k] = LdsElem<T>::get(sd, base + k * S);
        p[k] = k * S < lim ? fy[k] * fd[k] : 0.f;
      }
      const float dot = seg_allreduce<S>(tree_sum(p), OpAdd{});
#pragma unroll
      for (int k = 0; k < EPL; ++k)
        if (k * S < lim) LdsElem<T>::put(sy, base + k * S, fy[k] * (fd[k] - dot));
    }
    __syncthreads();
    if (full) {
      const rsrc_t ro = make_rsrc(dx + row0 * C, full_bytes);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int gv = tid + k * NT;
        if (gv < nvec) bstore128<kPolicyStream>(sy[gv], ro, voff, (uint32_t)k * NT * 16u);
      }
    } else {
      for (int i = tid; i < nrows * C; i += NT) E::store1(dx + row0 * C + i, LdsElem<T>::get(sy, i));
    }
    __syncthreads();  // the stages are refilled by the next step
  };

  u32x4 va[K], vb[K], ua[K], ub[K];
  if (chunk < nfull) load_full(chunk, va, vb);
  if (chunk + G < nfull) load_full(chunk + G, ua, ub);
  for (;;) {
    step(va, vb, chunk);
    chunk += G;
    if (chunk >= nchunks) break;
    step(ua, ub, chunk);
    chunk += G;
    if (chunk >= nchunks) break;
  }
}

// Sum of y_i * dy_i over the VE elements of a pair of vectors, in a fixed
// order (products, then a pairwise tree).
template <typename T>
__device__ __forceinline__ float vec_dot(u32x4 a, u32x4 b) {
  using E = Elem<T>;
  float fa[E::VE], fb[E::VE], p[E::VE];
  E::unpack(a, fa);
  E::unpack(b, fb);
#pragma unroll
  for (int i = 0; i < E::VE; ++i) p[i] = fa[i] * fb[i];
  return tree_sum(p);
}

template <typename T>
__device__ __forceinline__ u32x4 vec_dx(u32x4 a, u32x4 b, float dot) {
  using E = Elem<T>;
  float fa[E::VE], fb[E::VE], g[E::VE];
  E::unpack(a, fa);
  E::unpack(b, fb);
#pragma unroll
  for (int i = 0; i < E::VE; ++i) g[i] = fa[i] * (fb[i] - dot);
  return E::pack(g);
}

// ---------------------------------------------------------------------------
// Other rows: one workgroup of NT threads per row, persistent.  y, dy and dx
// must have the same address modulo 16 (the host checks), so one geometry
// (head elements, 16-byte body, tail) serves all three.
// ---------------------------------------------------------------------------
template <typename T, int NT, int NV>
__global__ __launch_bounds__(NT) void sm_bwd_row_kernel(const T* __restrict__ y,
                                                        const T* __restrict__ dy, int64_t B,
                                                        int C, T* __restrict__ dx) {
  using E = Elem<T>;
  constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0 && NW <= 16, "1 to 16 waves");
  __shared__ float red[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t voff = (uint32_t)tid * 16u;
  const int64_t G = gridDim.x;
  int64_t row = blockIdx.x;
  if (row >= B) return;  // whole workgroup

  auto body = [&](const T* base, int64_t r, bool exists) {
    const T* rp = base + r * C;
    const RowGeom g = row_geom(rp, C);
    return make_rsrc(rp + g.h, exists ? (uint32_t)g.nb * 16u : 0u);
  };

  u32x4 vy[NV], vd[NV];
  {
    const rsrc_t ry = body(y, row, true), rd = body(dy, row, true);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      vy[k] = bload128<kPolicyStream>(ry, voff, (uint32_t)k * NT * 16u);
      vd[k] = bload128<kPolicyStream>(rd, voff, (uint32_t)k * NT * 16u);
    }
  }

  for (int parity = 0;; parity ^= 1) {
    const T* yp = y + row * C;
    const T* dp = dy + row * C;
    T* op = dx + row * C;
    const RowGeom geo = row_geom(yp, C);
    const int nb = geo.nb;
    const rsrc_t ry = make_rsrc(yp + geo.h, (uint32_t)nb * 16u);
    const rsrc_t rd = make_rsrc(dp + geo.h, (uint32_t)nb * 16u);
    const rsrc_t ro = make_rsrc(op + geo.h, (uint32_t)nb * 16u);

    int xe = -1;  // this thread's edge element, if any
    if (tid < geo.h)
      xe = tid;
    else if (tid - geo.h < geo.ntail)
      xe = geo.tail0 + (tid - geo.h);
    const float ey = xe >= 0 ? E::load1(yp + xe) : 0.f;
    const float ed = xe >= 0 ? E::load1(dp + xe) : 0.f;

    // this thread's share of the dot: register slots (lanes past the row's
    // end read zeros through the buffer range), streamed vectors, edge
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (k * NT >= nb) continue;  // uniform
      acc += vec_dot<T>(vy[k], vd[k]);
    }
    for (int vi = NT * NV + tid; vi < nb; vi += NT) {
      const u32x4 a = bload128<kPolicyDefault>(ry, (uint32_t)vi * 16u, 0u);
      const u32x4 b = bload128<kPolicyDefault>(rd, (uint32_t)vi * 16u, 0u);
      acc += vec_dot<T>(a, b);
    }
    acc += ey * ed;

    float dot = wave_allreduce(acc, OpAdd{});
    if constexpr (NW > 1) {
      if (lane == 0) red[parity][tid >> 6] = dot;
      __syncthreads();
      const float pi = lane < NW ? red[parity][lane] : 0.f;
      dot = wave_uniform(seg_allreduce<16>(pi, OpAdd{}));
    }

    // dx from the registers; each slot is refilled with the next row's
    // vectors once its dx is packed (an empty resource after the last row)
    const int64_t next = row + G;
    const bool more = next < B;  // uniform
    const rsrc_t ryn = body(y, more ? next : row, more);
    const rsrc_t rdn = body(dy, more ? next : row, more);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      asm volatile("" : "+v"(vy[k]));
      asm volatile("" : "+v"(vd[k]));
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const bool in = k * NT < nb;  // uniform
      u32x4 packed;
      if (in) packed = vec_dx<T>(vy[k], vd[k], dot);
      vy[k] = bload128<kPolicyStream>(ryn, voff, (uint32_t)k * NT * 16u);
      vd[k] = bload128<kPolicyStream>(rdn, voff, (uint32_t)k * NT * 16u);
      __builtin_amdgcn_sched_barrier(0);
      if (in) bstore128<kPolicyStream>(packed, ro, voff, (uint32_t)k * NT * 16u);
    }
    for (int vi = NT * NV + tid; vi < nb; vi += NT) {
      const u32x4 a = bload128<kPolicyStream>(ry, (uint32_t)vi * 16u, 0u);
      const u32x4 b = bload128<kPolicyStream>(rd, (uint32_t)vi * 16u, 0u);
      bstore128<kPolicyStream>(vec_dx<T>(a, b, dot), ro, (uint32_t)vi * 16u, 0u);
    }
    if (xe >= 0) E::store1(op + xe, ey * (ed - dot));
    if (!more) break;
    row = next;
  }
}

}  // namespace ce
