// gfx950 kernels of the fused softmax cross-entropy path: short and tiny
// rows (path 1), one workgroup per row (paths 2 and 3), the loss reduction
// and the small helper kernels.  The per-row arithmetic and the row
// operations are in ce_rowops.h.
#pragma once

#include "ce_rowops.h"

namespace ce {

// ===========================================================================
// Path 1: short rows.  S lanes per row (S = 1..16), 256/S rows per group
// of a 256-thread workgroup and R groups per workgroup, all of whose loads
// are issued first.  Lane q of a segment holds the vectors q, q+S, ... of
// its row (VW elements each, EPL elements in all), so the lanes of a
// segment read consecutive addresses.  Max and sum are reduced across the
// segment with DPP; nothing goes through LDS.
// ===========================================================================

constexpr int kShortThreads = 256;

// GRAD false: the loss (or record) only; grad is not written (and may be
// null).
template <typename T, int S, int EPL, int VW, bool GRAD, int OP = kOpCE, int R = 1>
__global__ __launch_bounds__(kShortThreads) void ce_short_kernel(
    const T* __restrict__ logits, const int32_t* __restrict__ targets, int64_t B, int C,
    RowArgs rs, T* __restrict__ grad, float* __restrict__ loss_rows) {
  const float invB = row_invB(rs), gmul = grad_mul(rs);
  constexpr int RPG = kShortThreads / S;  // rows per group: one per segment
  constexpr int RPB = RPG * R;            // rows per workgroup: R groups
  constexpr int NVEC = EPL / VW;          // vector slots per lane
  static_assert(EPL % VW == 0, "EPL must be a multiple of VW");
  constexpr uint32_t ES = sizeof(T);

  const int tid = threadIdx.x;
  const int q = tid % S, seg = tid / S;
  const int64_t row0 = (int64_t)blockIdx.x * RPB;
  const int64_t nrows = (B - row0) < RPB ? (B - row0) : RPB;
  // the workgroup's rows, with the row strides (the host keeps these spans
  // below 2^31 bytes); lanes of rows past B read zeros and store nothing
  const rsrc_t rin = make_rsrc(logits + row0 * rs.ldz, (uint32_t)(((nrows - 1) * rs.ldz + C) * ES));
  const rsrc_t rout = make_rsrc(grad + row0 * rs.ldg, (uint32_t)(((nrows - 1) * rs.ldg + C) * ES));

  // every load of the R groups first: R rows' vectors in flight per lane
  float f[R][EPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t rowoff = (uint32_t)(r * RPG + seg) * (uint32_t)rs.ldz * ES;
#pragma unroll
    for (int j = 0; j < NVEC; ++j) {
      const int c0 = (j * S + q) * VW;
      float v[VW];
      if (c0 < C) {
        VecIO<T, VW>::load(rin, rowoff + (uint32_t)c0 * ES, v);
      } else {
#pragma unroll
        for (int w = 0; w < VW; ++w) v[w] = kNegInf;
      }
#pragma unroll
      for (int w = 0; w < VW; ++w) f[r][j * VW + w] = v[w];
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r * RPG + seg;
    const bool live = row < B;
    const RowTarget rt = live ? row_target<OP>(targets, row, C, rs) : RowTarget{-1, false, false};
    const int t = rt.t;
    const bool valid = live && rt.valid;
    // slot of the target in its owner lane: element c sits in vector c/VW,
    // lane (c/VW) % S, slot ((c/VW)/S)*VW + c%VW
    const int tq = t >= 0 ? (t / VW) % S : -1;
    const int tslot = t >= 0 ? ((t / VW) / S) * VW + t % VW : -1;
    const bool owner = (q == tq);
    // the target logit, from the owner lane's registers: a segment sum of
    // the owner's value and zeros is exact
    float own_zt = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) own_zt = (owner && i == tslot) ? f[r][i] : own_zt;
    const float zt = seg_allreduce<S>(own_zt, OpAdd{});

    // row max across the segment, then the sum with the target left out;
    // the terms are kept: scaled, they are the gradient
    const float m = seg_allreduce<S>(max_of(f[r]), OpMax{});
    const float cg = m * kLog2e;
    float e[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float x = (owner && i == tslot) ? kNegInf : f[r][i];
      e[i] = exp2_hw(__builtin_fmaf(x, kLog2e, -cg));
    }
    const float sx = seg_allreduce<S>(tree_sum(e), OpAdd{});
    const RowResult rr = row_finish<OP>(cg, sx, zt, valid, rt.ignored, invB, gmul);
    if (live && q == 0) store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);
    if constexpr (GRAD) {
      const uint32_t rowoff_g = (uint32_t)(r * RPG + seg) * (uint32_t)rs.ldg * ES;
#pragma unroll
      for (int j = 0; j < NVEC; ++j) {
        const int c0 = (j * S + q) * VW;
        if (c0 < C) {
          float g[VW];
#pragma unroll
          for (int w = 0; w < VW; ++w) {
            const int i = j * VW + w;
            g[w] = (owner && i == tslot) ? rr.gt : e[i] * rr.scale;
          }
          VecIO<T, VW>::store(rout, rowoff_g + (uint32_t)c0 * ES, g);
        }
      }
    }
  }
}

// ===========================================================================
// Path 1, rows of at most 64 bytes (fp32 C <= 16, bf16/fp16 C <= 32) with
// contiguous rows and 16-byte aligned arrays.  Each wave owns one chunk of
// 64 * R rows: at most R * 4 KB, and a whole number of 16-byte vectors
// (64 * C * size is a multiple of 16), so the wave reads it with whole
// 16-byte loads into its own LDS slot; each lane reduces R rows from LDS
// without any cross-lane step and writes their gradients back into the
// slot, and the chunk leaves with whole 16-byte stores.  A wave touches no
// other wave's slot, and one wave's LDS operations complete in issue
// order, so no workgroup barrier is needed.  The grid has one wave per
// chunk: the hardware dispatcher keeps every CU filled to the end (a
// persistent grid over the same chunks left CUs idle at the tail, and its
// barriers stalled all four waves of a workgroup on the slowest).  The
// last, partial chunk of a call is moved one element per lane instead.
// ===========================================================================
constexpr int kTinyThreads = 256;
constexpr int kTinyWaves = kTinyThreads / 64;
constexpr int kTinyRowBytes = 64;   // largest row

// Orders one wave's LDS accesses on either side (the hardware keeps them
// in order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
struct LdsElem;
template <>
struct LdsElem<float> {
  __device__ static __forceinline__ float get(const u32x4* st, int i) {
    return reinterpret_cast<const float*>(st)[i];
  }
  __device__ static __forceinline__ void put(u32x4* st, int i, float g) {
    reinterpret_cast<float*>(st)[i] = g;
  }
};
template <>
struct LdsElem<__bf16> {
  __device__ static __forceinline__ float get(const u32x4* st, int i) {
    return __builtin_bit_cast(float, (unsigned)reinterpret_cast<const unsigned short*>(st)[i] << 16);
  }
  __device__ static __forceinline__ void put(u32x4* st, int i, float g) {
    reinterpret_cast<unsigned short*>(st)[i] = (unsigned short)(pack_bf16x2(g, 0.f) & 0xffffu);
  }
};
template <>
struct LdsElem<_Float16> {
  __device__ static __forceinline__ float get(const u32x4* st, int i) {
    return f16lo((unsigned)reinterpret_cast<const unsigned short*>(st)[i]);
  }
  __device__ static __forceinline__ void put(u32x4* st, int i, float g) {
    reinterpret_cast<unsigned short*>(st)[i] = (unsigned short)(pack_f16x2(g, 0.f) & 0xffffu);
  }
};

// CMAX: the row length rounded up to 8, 12, 16 or 32 elements (at most 64
// bytes), the width of each lane's per-row arrays.  R: rows per lane.
template <typename T, int CMAX, int R, bool GRAD, int OP = kOpCE, bool PAD = false>
__global__ __launch_bounds__(kTinyThreads) void ce_tiny_kernel(const T* __restrict__ logits,
                                                               const int32_t* __restrict__ targets,
                                                               int64_t B, int C, RowArgs rs,
                                                               T* __restrict__ grad,
                                                               float* __restrict__ loss_rows) {
  using E = Elem<T>;
  constexpr int ES = sizeof(T), ROWS = 64 * R;                     // rows of a wave's chunk
  constexpr int K = (ROWS * CMAX * ES + 16 * 64 - 1) / (16 * 64);  // 16-byte loads per lane
  static_assert(CMAX * ES <= kTinyRowBytes, "row width");
  // PAD: rows of whole 32-bit words (C * size a multiple of 4) sit in LDS at
  // an odd stride of RS words, so that the lanes of a wave, each reading
  // its own row, hit different banks (at the row's own stride of 4, 8, 12
  // or 16 words they would share a few).
  constexpr int EPW = 4 / ES;                 // elements per word
  constexpr int RDMAX = CMAX / EPW;           // words of the widest row
  constexpr int SLOT = PAD ? (ROWS * (RDMAX | 1) + 3) / 4 : 64 * K;   // 16-byte units
  static_assert(!PAD || CMAX % EPW == 0, "whole words");
  __shared__ u32x4 slots[kTinyWaves][SLOT];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  u32x4* const stage = slots[wave];
  unsigned* const sw = reinterpret_cast<unsigned*>(stage);
  const float invB = row_invB(rs), gmul = grad_mul(rs);
  const uint32_t voff = (uint32_t)lane * 16u;
  const int64_t row0 = ((int64_t)blockIdx.x * kTinyWaves + wave) * ROWS;
  if (row0 >= B) return;                      // wave-uniform
  const bool full = row0 + ROWS <= B;
  const int nrows = full ? ROWS : (int)(B - row0);
  const uint32_t full_bytes = (uint32_t)(ROWS * C * ES);
  const int nvec = (int)(full_bytes / 16);    // 16-byte vectors of a full chunk
  // PAD: words per row (4, 8, 12 or 16: the host pads rows of a multiple of
  // 16 bytes) and the padded stride; word d of a chunk is word d - RD * (d /
  // RD) of row d / RD, with d / RD = high half of d * ceil(2^32 / RD),
  // exact since d * (ceil(2^32 / RD) * RD - 2^32) < 2^32 for d < ROWS * RD
  // <= 2^14
  const int RD = PAD ? C / EPW : 1;
  const int RS = RD | 1;
  const uint32_t magic =
      PAD ? (uint32_t)((0x100000000ull + (uint64_t)RD - 1u) / (uint64_t)RD) : 0u;
  static_assert(ROWS * RDMAX <= (1 << 14), "exact word division");
  auto word_slot = [&](int d) -> int {
    const int row = (int)(((uint64_t)(uint32_t)d * magic) >> 32);
    return row * RS + (d - row * RD);
  };
  // LDS index of element i of the chunk (rows of C elements)
  auto elem_slot = [&](int i) -> int {
    if constexpr (PAD) {
      const int row = i / C;
      return row * RS * EPW + (i - row * C);
    } else {
      return i;
    }
  };

  // the chunk's loads, and the targets of this lane's rows, all in flight
  // before the first is used
  u32x4 v[K];
  int32_t tg[R];
  if (full) {
    const rsrc_t r = make_rsrc(logits + row0 * C, full_bytes);
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = bload128<kPolicyStream>(r, voff, (uint32_t)k * 64u * 16u);
    if constexpr (OP != kOpSoftmax) {
#pragma unroll
      for (int j = 0; j < R; ++j) tg[j] = targets[row0 + lane + j * 64];
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int gv = lane + k * 64;
      if (gv >= nvec) continue;
      if constexpr (PAD) {
        sw[word_slot(4 * gv + 0)] = v[k].x;
        sw[word_slot(4 * gv + 1)] = v[k].y;
        sw[word_slot(4 * gv + 2)] = v[k].z;
        sw[word_slot(4 * gv + 3)] = v[k].w;
      } else {
        stage[gv] = v[k];
      }
    }
  } else {
    for (int i = lane; i < nrows * C; i += 64)
      LdsElem<T>::put(stage, elem_slot(i), E::load1(logits + row0 * C + i));
  }
  wave_lds_sync();

  // rows lane, lane + 64, ... of the chunk
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int lr = lane + j * 64;
    if (lr >= nrows) break;
    const int64_t row = row0 + lr;
    const RowTarget rt = full ? row_target_of<OP>(OP != kOpSoftmax ? tg[j] : -1, C, rs)
                              : row_target<OP>(targets, row, C, rs);
    const int t = rt.t;
    float f[CMAX];
    float m = kNegInf;
    if constexpr (PAD) {
#pragma unroll
      for (int k = 0; k < RDMAX; ++k) {
        const unsigned w = k < RD ? sw[lr * RS + k] : 0u;
#pragma unroll
        for (int q = 0; q < EPW; ++q) {
          const int c = k * EPW + q;
          f[c] = c < C ? widen_half<T>(w, q) : kNegInf;
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < CMAX; ++c) f[c] = c < C ? LdsElem<T>::get(stage, lr * C + c) : kNegInf;
    }
#pragma unroll
    for (int c = 0; c < CMAX; ++c) m = fmax2(m, f[c]);
    const float cg = m * kLog2e;
    float e[CMAX];
    float zt = 0.f;
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      zt = (c == t) ? f[c] : zt;
      e[c] = (c == t) ? 0.f : exp2_hw(__builtin_fmaf(f[c], kLog2e, -cg));
    }
    const float sx = tree_sum(e);
    const RowResult rr = row_finish<OP>(cg, sx, zt, rt.valid, rt.ignored, invB, gmul);
    store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);
    if constexpr (GRAD) {
      // the terms of the sum are the unnormalised softmax: scaled, they
      // are the gradient (the target's term was left out of the sum)
      float g[CMAX];
#pragma unroll
      for (int c = 0; c < CMAX; ++c) g[c] = c == t ? rr.gt : e[c] * rr.scale;
      if constexpr (PAD) {
#pragma unroll
        for (int k = 0; k < RDMAX; ++k)
          if (k < RD) sw[lr * RS + k] = pack_word<T>(&g[k * EPW]);
      } else {
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
          if (c < C) LdsElem<T>::put(stage, lr * C + c, g[c]);
      }
    }
  }
  if constexpr (GRAD) {
    wave_lds_sync();
    if (full) {
      const rsrc_t ro = make_rsrc(grad + row0 * C, full_bytes);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int gv = lane + k * 64;
        if (gv >= nvec) continue;
        u32x4 w;
        if constexpr (PAD) {
          w = u32x4{sw[word_slot(4 * gv + 0)], sw[word_slot(4 * gv + 1)],
                    sw[word_slot(4 * gv + 2)], sw[word_slot(4 * gv + 3)]};
        } else {
          w = stage[gv];
        }
        bstore128<kPolicyStream>(w, ro, voff, (uint32_t)k * 64u * 16u);
      }
    } else {
      for (int i = lane; i < nrows * C; i += 64)
        E::store1(grad + row0 * C + i, LdsElem<T>::get(stage, elem_slot(i)));
    }
  }
}

// ===========================================================================
// Path 1 (and path 2 up to 1024 elements), contiguous rows of more than 64
// bytes whose length in bytes is not a multiple of 16 (odd lengths, for
// example): the short kernel would read them with 8-, 4- or 2-byte loads,
// the row kernel its head and tail element by element.  Here a chunk
// of rows, which starts on a 16-byte boundary, is staged through LDS with
// whole 16-byte loads and stores as in the tiny kernel, and each row is
// reduced by a segment of S lanes as in the short kernel, lane q taking
// elements q, q+S, ... of its row from LDS.  A chunk holds as many whole
// passes of 256/S rows as fit kStagedChunkBytes (the count is set at run
// time from C, so short rows fill the chunk too); with rows of more than 32
// bytes that is fewer than 512 rows, so each thread loads at most two
// targets per chunk, with the chunk's data.  Rows of up to 128 bytes take 2
// lanes each, up to 64 elements (96 for 16-bit types) 4, 16-bit rows of 257
// to 1024 elements 32.  The workgroups are persistent
// and keep the loads of the next two chunks in flight in two register sets;
// the last, partial chunk of a call moves one element per thread.
// ===========================================================================
constexpr int kStagedThreads = 256;
constexpr int kStagedChunkBytes = 16384;  // K = 4 loads per thread and register set

// Rows per chunk for rows of C elements of es bytes: whole passes of rpp
// rows that fit `bytes` (a multiple of 8 rows, since rpp is, so every chunk
// starts on a 16-byte boundary; 0: not even one pass fits).  Whole passes
// measured faster than chunks filled to the last group of 8 rows, whose
// last pass leaves segments idle (fp32 rows of 33-91 elements 79-83 %
// of a copy's rate against 86-91 %).
__host__ __device__ constexpr int staged_rows_per_chunk(int C, int es, int rpp,
                                                        int bytes = kStagedChunkBytes) {
  return bytes / (rpp * C * es) * rpp;
}

// EPL: elements per lane, slots k = 0..EPL-1 at row offsets q + k*S
// (C <= S * EPL).  Every slot is read unconditionally (the stage has EPL * S
// elements of slack past the chunk, so a slot past its row's end reads the
// next row or the slack) and taken as -inf unless q + k*S < C; only the
// gradient's stores are predicated.  The target's LDS element is replaced
// by -inf once its value is read, so the terms leave it out of the sum with
// no test per element (the max takes z_t back in), and its gradient is
// written over the term's zero afterwards by the segment's first lane.
template <typename T, int S, int EPL, bool GRAD, int OP = kOpCE>
__global__ __launch_bounds__(kStagedThreads) void ce_staged_kernel(
    const T* __restrict__ logits, const int32_t* __restrict__ targets, int64_t B, int C,
    RowArgs rs, T* __restrict__ grad, float* __restrict__ loss_rows) {
  using E = Elem<T>;
  constexpr int ES = sizeof(T), NT = kStagedThreads;
  constexpr int RPP = NT / S;  // rows per pass: one per segment
  constexpr int K = kStagedChunkBytes / (16 * NT);
  constexpr int SLACK = (S * EPL * ES + 15) / 16;  // vectors past the chunk
  constexpr int TPT = 2;  // targets per thread and chunk: rows of more than 32 bytes
  static_assert(S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "segment size");
  static_assert(RPP % 8 == 0, "whole passes keep a chunk on a 16-byte boundary");
  __shared__ u32x4 stage[NT * K + SLACK];
  __shared__ int32_t stage_t[NT * TPT];
  const float invB = row_invB(rs), gmul = grad_mul(rs);
  const int tid = threadIdx.x, q = tid % S, seg = tid / S;
  const uint32_t voff = (uint32_t)tid * 16u;
  // C * size > 32 bytes: fewer than 512 rows per chunk, at least one pass
  const int ROWS = staged_rows_per_chunk(C, ES, RPP);
  const int64_t nchunks = (B + ROWS - 1) / ROWS;
  const int64_t nfull = B / ROWS;
  const uint32_t full_bytes = (uint32_t)(ROWS * C * ES);
  const int nvec = (int)(full_bytes / 16);
  const int lim = C - q;  // slot k of this lane lies in the row iff k * S < lim
  int64_t chunk = blockIdx.x;
  if (chunk >= nchunks) return;  // whole workgroup

  // a full chunk's loads, and the targets of its rows tid and tid + NT (if
  // any)
  auto load_full = [&](int64_t ch, u32x4 (&v)[K], int32_t (&tg)[TPT]) {
    const rsrc_t r = make_rsrc(logits + ch * ROWS * C, full_bytes);
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = bload128<kPolicyStream>(r, voff, (uint32_t)k * NT * 16u);
    if constexpr (OP != kOpSoftmax) {
#pragma unroll
      for (int j = 0; j < TPT; ++j)
        if (tid + j * NT < ROWS) tg[j] = targets[ch * ROWS + tid + j * NT];
    }
  };
  const int64_t G = gridDim.x;
  auto step = [&](u32x4 (&r)[K], int32_t (&tg)[TPT], int64_t ch) {
    const int64_t row0 = ch * ROWS;
    const bool full = ch < nfull;
    const int nrows = full ? ROWS : (int)(B - row0);
    if (full) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int gv = tid + k * NT;
        if (gv < nvec) stage[gv] = r[k];
      }
#pragma unroll
      for (int j = 0; j < TPT; ++j)
        if (tid + j * NT < ROWS) stage_t[tid + j * NT] = tg[j];
    } else {
      for (int i = tid; i < nrows * C; i += NT)
        LdsElem<T>::put(stage, i, E::load1(logits + row0 * C + i));
      if constexpr (OP != kOpSoftmax) {
#pragma unroll
        for (int j = 0; j < TPT; ++j)
          if (tid + j * NT < nrows) stage_t[tid + j * NT] = targets[row0 + tid + j * NT];
      }
    }
    __syncthreads();
    if (ch + 2 * G < nfull) load_full(ch + 2 * G, r, tg);

#pragma unroll 1
    for (int lr = seg; lr < nrows; lr += RPP) {  // whole segments
      const int64_t row = row0 + lr;
      const RowTarget rt = row_target_of<OP>(OP != kOpSoftmax ? stage_t[lr] : -1, C, rs);
      const int t = rt.t;
      const int base = lr * C + q;  // this lane's element of slot k: base + k * S
      // the target logit (every lane of the segment reads it), then -inf in
      // its place
      float zt = 0.f;
      if (t >= 0) {
        zt = LdsElem<T>::get(stage, lr * C + t);
        if (q == 0) LdsElem<T>::put(stage, lr * C + t, kNegInf);
      }
      float f[EPL];
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        const float x = LdsElem<T>::get(stage, base + k * S);
        f[k] = k * S < lim ? x : kNegInf;
      }
      float m = max_of(f);
      m = seg_allreduce<S>(m, OpMax{});
      if (t >= 0) m = fmax2(m, zt);
      const float cg = m * kLog2e;
      // the terms, in place
#pragma unroll
      for (int k = 0; k < EPL; ++k) f[k] = exp2_hw(__builtin_fmaf(f[k], kLog2e, -cg));
      const float sx = seg_allreduce<S>(tree_sum(f), OpAdd{});
      const RowResult rr = row_finish<OP>(cg, sx, zt, rt.valid, rt.ignored, invB, gmul);
      if (q == 0) store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);
      if constexpr (GRAD) {
        // the terms, scaled, are the gradient; the target's (zero) is then
        // overwritten with g_t, later in the same wave's program order
#pragma unroll
        for (int k = 0; k < EPL; ++k)
          if (k * S < lim) LdsElem<T>::put(stage, base + k * S, f[k] * rr.scale);
        if (t >= 0 && q == 0) LdsElem<T>::put(stage, lr * C + t, rr.gt);
      }
    }
    if constexpr (GRAD) {
      __syncthreads();
      if (full) {
        const rsrc_t ro = make_rsrc(grad + row0 * C, full_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int gv = tid + k * NT;
          if (gv < nvec) bstore128<kPolicyStream>(stage[gv], ro, voff, (uint32_t)k * NT * 16u);
        }
      } else {
        for (int i = tid; i < nrows * C; i += NT)
          E::store1(grad + row0 * C + i, LdsElem<T>::get(stage, i));
      }
    }
    __syncthreads();  // the stage is refilled by the next step
  };

  u32x4 v[K], u[K];
  int32_t tv[TPT] = {-1, -1}, tu[TPT] = {-1, -1};
  if (chunk < nfull) load_full(chunk, v, tv);
  if (chunk + G < nfull) load_full(chunk + G, u, tu);
  for (;;) {
    step(v, tv, chunk);
    chunk += G;
    if (chunk >= nchunks) break;
    step(u, tu, chunk);
    chunk += G;
    if (chunk >= nchunks) break;
  }
}

// ===========================================================================
// Paths 2 and 3: one workgroup of NT threads per row at a time.  The row's
// aligned body is split into 16-byte vectors; thread i holds vectors i,
// i+NT, ..., i+(NV-1)NT in registers (NV*16 bytes per thread).  Vectors
// beyond NT*NV (path 3) are streamed: folded into the online state on the
// first read and read again for the gradient.  The up to 2*(VE-1) elements
// before the first 16-byte boundary and after the last one are handled one
// per thread.
//
// The workgroups are persistent: workgroup w takes rows w, w+G, w+2G, ...
// (G = gridDim.x, sized to the resident capacity of the GPU) and the
// per-row work is software-pipelined across rows:
//   Phase B: each thread folds its vectors of row r into an online (c, s)
//            state as they arrive, with the target element left out of s.
//   Combine: (c, s) is reduced over the wave with DPP, the waves' pairs go
//            through LDS (double-buffered by row parity, so one barrier per
//            row suffices), and every wave combines them in the same order.
//   Phase C: for each register slot, the vector of row r is widened, the
//            slot is immediately refilled with the load of the same slot of
//            row r+G, and the gradient of row r is written with streaming
//            stores.  The loads of the next row are in flight while this
//            row's gradient is formed and written.
// ===========================================================================
struct RowGeom {
  int h;       // elements before the first ALIGN-byte boundary
  int nb;      // 16-byte vectors from there on
  int tail0;   // first element after them
  int ntail;   // elements after them
};

// Row-relative indices fit in 32 bits: C <= 2^28.  The body starts at the
// first ALIGN-byte boundary of the row (ALIGN a power of two >= 16).
template <typename T, int ALIGN = 16>
__device__ __forceinline__ RowGeom row_geom(const T* rp, int C) {
  constexpr int VE = Elem<T>::VE;
  static_assert(ALIGN >= 16 && (ALIGN & (ALIGN - 1)) == 0, "alignment");
  RowGeom g;
  const uint32_t mis = (uint32_t)((uintptr_t)rp & (uint32_t)(ALIGN - 1));
  g.h = mis ? (int)((ALIGN - mis) / sizeof(T)) : 0;
  if (g.h > C) g.h = C;
  g.nb = (C - g.h) / VE;
  g.tail0 = g.h + g.nb * VE;
  g.ntail = C - g.tail0;
  return g;
}

// GRAD false: the loss (or record) only; grad is not written (and may be
// null), and the streamed part of a long row is read once.
template <typename T, int NT, int NV, bool GRAD, int OP = kOpCE>
__global__ __launch_bounds__(NT) void ce_row_kernel(const T* __restrict__ logits,
                                                    const int32_t* __restrict__ targets,
                                                    int64_t B, int C, RowArgs rs,
                                                    T* __restrict__ grad,
                                                    float* __restrict__ loss_rows) {
  const float invB = row_invB(rs), gmul = grad_mul(rs);
  using E = Elem<T>;
  constexpr int VE = E::VE;
  constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0 && NW <= 16, "1 to 16 waves");
  __shared__ float red_c[2][NW], red_s[2][NW];
  // fp32: keep the register slots' terms for the gradient in place of z
  // (no extra registers).  Keeping them for 16-bit types needs a float copy
  // of every slot; on 2048-wide bf16 rows it cost as much occupancy as it
  // saved arithmetic, so they recompute.
  constexpr bool kKeep = sizeof(T) == 4;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t voff = (uint32_t)tid * 16u;
  const int64_t G = gridDim.x;
  int64_t row = blockIdx.x;
  if (row >= B) return;  // whole workgroup

  // Phase A of the first row: issue every register load
  u32x4 v[NV];
  {
    const T* rp = logits + row * rs.ldz;
    const RowGeom geo = row_geom(rp, C);
    const rsrc_t rin = make_rsrc(rp + geo.h, (uint32_t)geo.nb * 16u);
#pragma unroll
    for (int k = 0; k < NV; ++k)
      v[k] = bload128<kPolicyStream>(rin, voff, (uint32_t)k * NT * 16u);
  }

  for (int parity = 0;; parity ^= 1) {
    const T* rp = logits + row * rs.ldz;
    T* gp = grad + row * rs.ldg;
    const RowGeom geo = row_geom(rp, C);
    const int nb = geo.nb;
    const rsrc_t rin = make_rsrc(rp + geo.h, (uint32_t)nb * 16u);
    const rsrc_t rout = make_rsrc(gp + geo.h, (uint32_t)nb * 16u);

    const RowTarget rt = row_target<OP>(targets, row, C, rs);
    const int t = rt.t;
    const bool valid = rt.valid;
    // where the target lives: body vector tv (element tj), or an edge element
    const int tb = t - geo.h;
    const bool t_in_body = t >= 0 && tb >= 0 && tb < nb * VE;
    const int tv = t_in_body ? tb / VE : -1;                                  // uniform
    const int tj = t_in_body ? tb % VE : -1;                                  // uniform
    const int own_k = (t_in_body && tv < NT * NV) ? tv / NT : -1;             // uniform
    const bool own_thread = t_in_body && (tv % NT) == tid;

    int xe = -1;  // this thread's edge element, if any
    if (tid < geo.h)
      xe = tid;
    else if (tid - geo.h < geo.ntail)
      xe = geo.tail0 + (tid - geo.h);
    const float xs = xe >= 0 ? E::load1(rp + xe) : kNegInf;
    const float zt = t >= 0 ? E::load1(rp + t) : 0.f;

    // Phase B: online max / sum-exp over the thread's elements.  With kKeep,
    // each register slot's terms 2^(z log2e - ck[k]) replace z (ck[k] the
    // running max after slot k); the gradient is then one multiply per
    // element.
    float c = kLowest, s = 0.f;
    float ck[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int base = k * NT;
      ck[k] = c;
      if (base >= nb) continue;  // uniform: no vector of this slot is in the row
      float f[VE];
      E::unpack(v[k], f);
      if (base + NT > nb) {
        const bool ok = tid < nb - base;
#pragma unroll
        for (int i = 0; i < VE; ++i) f[i] = ok ? f[i] : kNegInf;
      }
      const float vm = max_of(f);
      if (k == own_k && own_thread) {
#pragma unroll
        for (int i = 0; i < VE; ++i) f[i] = (i == tj) ? kNegInf : f[i];
      }
      if constexpr (GRAD && kKeep) {
        float e[VE];
        online_fold_e(c, s, vm, f, e);
        ck[k] = c;
        v[k] = as_u32(f32x4{e[0], e[1], e[2], e[3]});
      } else {
        online_fold(c, s, vm, f);
      }
    }
    // path 3: the part of the row beyond the registers, streamed
    for (int vi = NT * NV + tid; vi < nb; vi += NT) {
      const u32x4 w = bload128<kPolicyDefault>(rin, (uint32_t)vi * 16u, 0u);
      float f[VE];
      E::unpack(w, f);
      const float vm = max_of(f);
      if (vi == tv) {
#pragma unroll
        for (int i = 0; i < VE; ++i) f[i] = (i == tj) ? kNegInf : f[i];
      }
      online_fold(c, s, vm, f);
    }
    if (xe >= 0) {
      const float one[1] = {(xe == t) ? kNegInf : xs};
      online_fold(c, s, xs, one);
    }

    // Combine: wave, then workgroup, in a fixed order
    const float cw = wave_allreduce(c, OpMax{});
    const float sw = wave_allreduce(s * exp2_hw(c - cw), OpAdd{});
    float cg, sx;
    if constexpr (NW == 1) {
      cg = cw;
      sx = sw;
    } else {
      const int wv = tid >> 6;
      if (lane == 0) {
        red_c[parity][wv] = cw;
        red_s[parity][wv] = sw;
      }
      __syncthreads();
      const float ci = lane < NW ? red_c[parity][lane] : kLowest;
      const float si = lane < NW ? red_s[parity][lane] : 0.f;
      cg = wave_uniform(seg_allreduce<16>(ci, OpMax{}));
      sx = wave_uniform(seg_allreduce<16>(si * exp2_hw(ci - cg), OpAdd{}));
    }
    const RowResult rr = row_finish<OP>(cg, sx, zt, valid, rt.ignored, invB, gmul);
    if (tid == 0) store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);

    // Phase C: gradient from the registers; each slot is refilled with the
    // next row's vector as soon as it has been widened.  After the last row
    // the refill goes through an empty buffer resource: it returns zeros
    // without a memory access.
    const int64_t next = row + G;
    const bool more = next < B;  // uniform
    const T* rpn = logits + (more ? next : row) * rs.ldz;
    const RowGeom geon = row_geom(rpn, C);
    const rsrc_t rinn = make_rsrc(rpn + geon.h, more ? (uint32_t)geon.nb * 16u : 0u);
    // The empty asm makes each packed vector opaque here, so the compiler
    // widens it again instead of keeping phase B's widened copy alive
    // (twice the registers for bf16).
#pragma unroll
    for (int k = 0; k < NV; ++k) asm volatile("" : "+v"(v[k]));
    if constexpr (!GRAD) {
#pragma unroll
      for (int k = 0; k < NV; ++k) v[k] = bload128<kPolicyStream>(rinn, voff, (uint32_t)k * NT * 16u);
      if (!more) break;
      row = next;
      continue;
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int base = k * NT;
      // the gradient of this slot is packed before the slot is refilled, so
      // the refill can reuse the slot's registers
      u32x4 packed;
      if (base < nb) {  // uniform
        float g[VE];
        if constexpr (kKeep) {
          const float factor = exp2_hw(ck[k] - cg) * rr.scale;
          const f32x4 e = as_f32(v[k]);
          g[0] = e.x * factor;
          g[1] = e.y * factor;
          g[2] = e.z * factor;
          g[3] = e.w * factor;
        } else {
          float f[VE];
          E::unpack(v[k], f);
#pragma unroll
          for (int i = 0; i < VE; ++i) g[i] = exp2_hw(__builtin_fmaf(f[i], kLog2e, -cg)) * rr.scale;
        }
        if (k == own_k && own_thread) {
#pragma unroll
          for (int i = 0; i < VE; ++i) g[i] = (i == tj) ? rr.gt : g[i];
        }
        packed = E::pack(g);
      }
      v[k] = bload128<kPolicyStream>(rinn, voff, (uint32_t)k * NT * 16u);
      if (base < nb) bstore128<kPolicyStream>(packed, rout, voff, (uint32_t)k * NT * 16u);
      // keep slot order: a later slot's refill must not be hoisted above
      // this slot's use of its registers
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int vi = NT * NV + tid; vi < nb; vi += NT) {
      const u32x4 w = bload128<kPolicyStream>(rin, (uint32_t)vi * 16u, 0u);
      float f[VE], g[VE];
      E::unpack(w, f);
#pragma unroll
      for (int i = 0; i < VE; ++i) g[i] = exp2_hw(__builtin_fmaf(f[i], kLog2e, -cg)) * rr.scale;
      if (vi == tv) {
#pragma unroll
        for (int i = 0; i < VE; ++i) g[i] = (i == tj) ? rr.gt : g[i];
      }
      bstore128<kPolicyStream>(E::pack(g), rout, (uint32_t)vi * 16u, 0u);
    }
    if (xe >= 0) {
      const float g = (xe == t) ? rr.gt : exp2_hw(__builtin_fmaf(xs, kLog2e, -cg)) * rr.scale;
      E::store1(gp + xe, g);
    }
    if (!more) break;
    row = next;
  }
}

// ===========================================================================
// Path 2 for rows of more than 8192 16-byte vectors (bf16 C > 65528, fp32
// C > 32764): the row kernel above with the next row's first PF slots
// (PF*16 KB) prefetched into LDS by direct-to-LDS buffer loads.
//
// Loads and stores retire in order on this GPU, so a wait for a load also
// waits for every store issued before it.  The prefix of row r+1 is issued
// right after row r's prefix has been copied out of LDS, before any store of
// row r, so waiting for it never waits for stores; only the NV-PF register
// slots are still refilled during phase C.  The copy of the prefix into the
// registers costs one LDS read per element.
//
// Every wait below is a fixed vmcnt, so every load and store in the loop is
// issued unconditionally (buffer-resource bounds make the ones outside the
// row no-ops), and the first row is preceded by the same number of
// operations as a steady-state row.  Wave 0 also stores the per-row loss and
// the edge elements; those are left out of the count, which only makes wave
// 0 wait slightly longer.
// ===========================================================================
template <typename T>
__device__ __forceinline__ float bload_elem(rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ float bload_elem<float>(rsrc_t r, uint32_t off) {
  const unsigned d = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicyDefault);
  return __builtin_bit_cast(float, d);
}
template <>
__device__ __forceinline__ float bload_elem<__bf16>(rsrc_t r, uint32_t off) {
  const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, kPolicyDefault);
  return __builtin_bit_cast(float, (unsigned)h << 16);
}
template <>
__device__ __forceinline__ float bload_elem<_Float16>(rsrc_t r, uint32_t off) {
  const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, kPolicyDefault);
  return f16lo((unsigned)h);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt vmcnt(N) only (expcnt, lgkmcnt left at their maxima), as asm
// with a memory clobber so no memory access moves across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <typename T, int NV, int PF, int OP = kOpCE>
__global__ __launch_bounds__(1024) void ce_row_lds_kernel(const T* __restrict__ logits,
                                                          const int32_t* __restrict__ targets,
                                                          int64_t B, int C, RowArgs rs,
                                                          T* __restrict__ grad,
                                                          float* __restrict__ loss_rows) {
  const float invB = row_invB(rs), gmul = grad_mul(rs);
  using E = Elem<T>;
  constexpr int NT = 1024, NW = 16, VE = E::VE, ES = sizeof(T);
  static_assert(PF >= 1 && PF < NV, "prefetch slots");
  // VMEM operations one wave issues after a row's prefix DMA and before the
  // wait for it: the previous row's phase C (refill load + store per
  // register slot, store per prefetched slot) and this row's two edge loads.
  constexpr int kAfterDma = 2 * (NV - PF) + PF + 2;
  __shared__ u32x4 stage[PF * NT];
  __shared__ float red_c[2][NW], red_s[2][NW];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t voff = (uint32_t)tid * 16u;
  const int64_t G = gridDim.x;
  int64_t row = blockIdx.x;
  if (row >= B) return;

  auto body_rsrc = [&](int64_t r, bool exists) {
    const T* rp = logits + r * rs.ldz;
    const RowGeom g = row_geom(rp, C);
    return make_rsrc(rp + g.h, exists ? (uint32_t)g.nb * 16u : 0u);
  };
  auto dma_prefix = [&](rsrc_t rs) {
#pragma unroll
    for (int p = 0; p < PF; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&stage[p * NT + wv * 64], 16, voff,
                                               (uint32_t)p * NT * 16u, 0, kPolicyStream);
  };

  u32x4 v[NV];
  // prologue: the same VMEM sequence as a steady-state row, so the wait
  // counts below hold for the first row too
  {
    dma_prefix(body_rsrc(row, true));
    const rsrc_t rin = body_rsrc(row, true);
    const rsrc_t none = make_rsrc(grad, 0u);
    // distinct (out-of-range) offsets keep the compiler from merging them
#pragma unroll
    for (int k = PF; k < NV; ++k) {
      v[k] = bload128<kPolicyStream>(rin, voff, (uint32_t)k * NT * 16u);
      bstore128<kPolicyStream>(u32x4{0, 0, 0, 0}, none, voff, (uint32_t)k * NT * 16u);
    }
#pragma unroll
    for (int k = 0; k < PF; ++k)
      bstore128<kPolicyStream>(u32x4{0, 0, 0, 0}, none, voff, (uint32_t)k * NT * 16u);
  }

  for (int parity = 0;; parity ^= 1) {
    const T* rp = logits + row * rs.ldz;
    T* gp = grad + row * rs.ldg;
    const RowGeom geo = row_geom(rp, C);
    const int nb = geo.nb;
    const rsrc_t rout = make_rsrc(gp + geo.h, (uint32_t)nb * 16u);
    const rsrc_t rrow = make_rsrc(rp, (uint32_t)C * ES);

    const RowTarget rt = row_target<OP>(targets, row, C, rs);
    const int t = rt.t;
    const bool valid = rt.valid;
    const int tb = t - geo.h;
    const bool t_in_body = t >= 0 && tb >= 0 && tb < nb * VE;
    const int tv = t_in_body ? tb / VE : -1;
    const int tj = t_in_body ? tb % VE : -1;
    const int own_k = (t_in_body && tv < NT * NV) ? tv / NT : -1;
    const bool own_thread = t_in_body && (tv % NT) == tid;

    int xe = -1;
    if (tid < geo.h)
      xe = tid;
    else if (tid - geo.h < geo.ntail)
      xe = geo.tail0 + (tid - geo.h);
    // step 1: edge loads, unconditional (an absent element reads past the row: 0)
    const float xs_raw = bload_elem<T>(rrow, (uint32_t)(xe >= 0 ? xe : C) * ES);
    const float zt_raw = bload_elem<T>(rrow, (uint32_t)(t >= 0 ? t : C) * ES);

    // step 2: this row's prefix is in LDS once everything issued before the
    // DMA has completed
    wait_vmcnt<kAfterDma>();
    // step 3: prefix slots LDS -> registers
#pragma unroll
    for (int p = 0; p < PF; ++p) v[p] = stage[p * NT + tid];
    wait_lgkm0();
    // step 4: prefetch the next row's prefix (issued before this row's stores)
    const int64_t next = row + G;
    const bool more = next < B;
    const int64_t nrow = more ? next : row;
    const rsrc_t rinn = body_rsrc(nrow, more);
    dma_prefix(rinn);

    const float xs = xe >= 0 ? xs_raw : kNegInf;
    const float zt = t >= 0 ? zt_raw : 0.f;

    // step 5: phase B
    float c = kLowest, s = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int base = k * NT;
      if (base >= nb) continue;
      float f[VE];
      E::unpack(v[k], f);
      if (base + NT > nb) {
        const bool ok = tid < nb - base;
#pragma unroll
        for (int i = 0; i < VE; ++i) f[i] = ok ? f[i] : kNegInf;
      }
      const float vm = max_of(f);
      if (k == own_k && own_thread) {
#pragma unroll
        for (int i = 0; i < VE; ++i) f[i] = (i == tj) ? kNegInf : f[i];
      }
      online_fold(c, s, vm, f);
    }
    if (xe >= 0) {
      const float one[1] = {(xe == t) ? kNegInf : xs};
      online_fold(c, s, xs, one);
    }

    // step 6: combine
    const float cw = wave_allreduce(c, OpMax{});
    const float sw = wave_allreduce(s * exp2_hw(c - cw), OpAdd{});
    if (lane == 0) {
      red_c[parity][wv] = cw;
      red_s[parity][wv] = sw;
    }
    // LDS-only barrier: the exchange goes through LDS, so only LDS traffic
    // has to complete first (a full __syncthreads would also wait for the
    // next row's prefetch)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const float ci = lane < NW ? red_c[parity][lane] : kLowest;
    const float si = lane < NW ? red_s[parity][lane] : 0.f;
    const float cg = wave_uniform(seg_allreduce<16>(ci, OpMax{}));
    const float sx = wave_uniform(seg_allreduce<16>(si * exp2_hw(ci - cg), OpAdd{}));
    const RowResult rr = row_finish<OP>(cg, sx, zt, valid, rt.ignored, invB, gmul);

    // step 7: phase C; register-only slots first (each refilled with the
    // next row), then the prefetched slots
#pragma unroll
    for (int k = 0; k < NV; ++k) asm volatile("" : "+v"(v[k]));
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int k = (j + PF) % NV;
      float f[VE], g[VE];
      E::unpack(v[k], f);
#pragma unroll
      for (int i = 0; i < VE; ++i) g[i] = exp2_hw(__builtin_fmaf(f[i], kLog2e, -cg)) * rr.scale;
      if (k == own_k && own_thread) {
#pragma unroll
        for (int i = 0; i < VE; ++i) g[i] = (i == tj) ? rr.gt : g[i];
      }
      const u32x4 packed = E::pack(g);
      if (k >= PF) v[k] = bload128<kPolicyStream>(rinn, voff, (uint32_t)k * NT * 16u);
      // the scheduling barrier sits before the store: placed right after a
      // store wider than 8 bytes it hides the store from the compiler's
      // hazard check, and a following write to the store's data registers
      // then lands without the wait states the hardware needs
      __builtin_amdgcn_sched_barrier(0);
      bstore128<kPolicyStream>(packed, rout, voff, (uint32_t)k * NT * 16u);
    }
    if (tid == 0) store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);
    if (xe >= 0) {
      const float g = (xe == t) ? rr.gt : exp2_hw(__builtin_fmaf(xs, kLog2e, -cg)) * rr.scale;
      E::store1(gp + xe, g);
    }
    if (!more) {
      // no LDS write may still be in flight when the workgroup's LDS is
      // handed to the next workgroup
      wait_vmcnt<0>();
      break;
    }
    row = next;
  }
}


// ===========================================================================
// Loss reduction: a fixed two-level tree.  Workgroup g of the first level
// sums the contiguous range [g*chunk, (g+1)*chunk) of the input (chunk a
// multiple of kReduceRound); in each round of kReduceRound values, thread i
// loads values i, i+256, ..., i+1792 of the round (eight 4-byte loads, all
// in flight at once; values past the range read as 0 through the buffer
// resource, and adding +0 leaves a sum unchanged) and adds each into its own
// accumulator, so every accumulator takes its values in index order.  The
// workgroup combines its threads with DPP/ds_swizzle and four LDS slots in
// a fixed order.  The second level is ce_reduce_one_kernel over the first
// level's partial sums.  Nothing depends on timing, so the result is
// reproducible bit for bit.
// ===========================================================================
constexpr int kReduceThreads = 256;
constexpr int kReduceLoads = 8;                               // per thread per round
constexpr int kReduceRound = kReduceThreads * kReduceLoads;   // values per round

__device__ __forceinline__ float block_sum_256(float v) {
  __shared__ float part[kReduceThreads / 64];
  const float w = wave_allreduce(v, OpAdd{});
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = w;
  __syncthreads();
  return (part[0] + part[1]) + (part[2] + part[3]);
}

__global__ __launch_bounds__(kReduceThreads) void ce_reduce_kernel(const float* __restrict__ in,
                                                                   int64_t n, int64_t chunk,
                                                                   float* __restrict__ out) {
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t len = (lo + chunk) < n ? chunk : n - lo;     // <= chunk < 2^30 (host check)
  const rsrc_t r = make_rsrc(in + lo, (uint32_t)len * 4u);
  const int rounds = (int)(chunk / kReduceRound);
  const uint32_t voff = threadIdx.x * 4u;
  float a[kReduceLoads];
#pragma unroll
  for (int k = 0; k < kReduceLoads; ++k) a[k] = 0.f;
  for (int it = 0; it < rounds; ++it) {
    float x[kReduceLoads];
#pragma unroll
    for (int k = 0; k < kReduceLoads; ++k)
      x[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           r, (int)voff, (it * kReduceRound + k * kReduceThreads) * 4,
                                           kPolicyDefault));
#pragma unroll
    for (int k = 0; k < kReduceLoads; ++k) a[k] = a[k] + x[k];
  }
  const float tot = block_sum_256(((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7])));
  if (threadIdx.x == 0) out[blockIdx.x] = tot;
}

// One workgroup of 1024 threads sums up to kReduceOneMax values with one
// round of loads: thread i reads values i, i + 1024, ... (at most 16, all in
// flight at once; the buffer's range returns 0 past n, and adding +0 leaves
// a sum unchanged) and adds them in index order; the waves' sums are
// combined across lanes in a fixed order and the 16 wave sums by a fixed
// pairwise tree.  Used for the whole sum up to kReduceOneMax rows and for
// the second level over the first level's partial sums.
constexpr int kReduceOneThreads = 1024;
constexpr int kReduceOneSlots = 16;
constexpr int kReduceOneMax = kReduceOneThreads * kReduceOneSlots;

__global__ __launch_bounds__(kReduceOneThreads) void ce_reduce_one_kernel(
    const float* __restrict__ in, int n, float* __restrict__ out) {
  __shared__ float part[kReduceOneThreads / 64];
  const int tid = threadIdx.x;
  const rsrc_t r = make_rsrc(in, (uint32_t)n * 4u);
  float v[kReduceOneSlots];
#pragma unroll
  for (int k = 0; k < kReduceOneSlots; ++k) {
    v[k] = 0.f;
    if (k * kReduceOneThreads < n)  // uniform
      v[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           r, (tid + k * kReduceOneThreads) * 4, 0, kPolicyDefault));
  }
  float a = v[0];
#pragma unroll
  for (int k = 1; k < kReduceOneSlots; ++k) a = a + v[k];
  const float w = wave_allreduce(a, OpAdd{});
  if ((tid & 63) == 0) part[tid >> 6] = w;
  __syncthreads();
  if (tid == 0) {
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = part[i];
    *out = tree_sum(t);
  }
}

// ===========================================================================
// Rows kept by ignore_index: the number of targets that differ from it.  A
// workgroup of 1024 threads reads rounds of 16384 targets, each thread 16
// of them at once (4-byte buffer loads, index-checked against B), and sums
// its threads' counts in integers.  With ONE, a single workgroup covers all
// B rows and stores the total; otherwise ce_set_u32_kernel zeroes the count
// first on the same stream and every workgroup adds its total with one
// integer atomic (an integer total does not depend on the order of the
// additions).
// ===========================================================================
constexpr int kCountThreads = 1024;
constexpr int kCountLoads = 16;                              // per thread per round
constexpr int kCountRound = kCountThreads * kCountLoads;     // targets per round

template <bool ONE>
__global__ __launch_bounds__(kCountThreads) void ce_count_kept_kernel(
    const int32_t* __restrict__ targets, int64_t B, int32_t ignore, uint32_t* __restrict__ count) {
  __shared__ uint32_t part[kCountThreads / 64];
  const int tid = threadIdx.x;
  uint32_t n = 0;
  const int64_t stride = (int64_t)gridDim.x * kCountRound;
  for (int64_t base = (int64_t)blockIdx.x * kCountRound; base < B; base += stride) {
    const int len = B - base < kCountRound ? (int)(B - base) : kCountRound;
    const rsrc_t r = make_rsrc(targets + base, (uint32_t)len * 4u);
    int32_t x[kCountLoads];
#pragma unroll
    for (int k = 0; k < kCountLoads; ++k)
      x[k] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r, tid * 4, k * kCountThreads * 4,
                                                           kPolicyDefault);
#pragma unroll
    for (int k = 0; k < kCountLoads; ++k)
      n += (tid + k * kCountThreads < len && x[k] != ignore) ? 1u : 0u;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n += (uint32_t)__shfl_xor((int)n, m, 64);
  if ((tid & 63) == 0) part[tid >> 6] = n;
  __syncthreads();
  if (tid == 0) {
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < kCountThreads / 64; ++i) tot += part[i];
    if constexpr (ONE)
      *count = tot;
    else if (tot != 0)
      atomicAdd(count, tot);
  }
}
__global__ __launch_bounds__(64) void ce_set_u32_kernel(uint32_t* __restrict__ p, uint32_t v) {
  if (threadIdx.x == 0) *p = v;
}

// ===========================================================================
// Backward broadcast-scale: g *= *scale in place over n elements (the
// gradient was formed in the forward pass; the backward multiplies it by
// the upstream gradient of the loss, a device scalar).  Every workgroup
// first reads the scalar and returns at once when it is exactly 1, so the
// common case moves no gradient bytes (about 16 us of launches at 2 GB of
// bf16).  The grid has one workgroup per chunk of 8192 16-byte vectors of
// the aligned body, the fastest streaming pattern measured (a grid capped
// at 2048 workgroups halved the no-op time and cost 3.5 % on a full pass);
// workgroup 0 also takes the elements before the first 16-byte boundary
// and after the last.
// ===========================================================================
constexpr int kScaleThreads = 1024;
constexpr int kScaleSlots = 8;

template <typename T>
__global__ __launch_bounds__(kScaleThreads) void ce_scale_kernel(T* __restrict__ g, int64_t n,
                                                                 const float* __restrict__ scale) {
  using E = Elem<T>;
  constexpr int VE = E::VE, ES = sizeof(T);
  const float sc = *scale;
  if (sc == 1.0f) return;
  const uint32_t mis = (uint32_t)((uintptr_t)g & 15u);
  int64_t h = mis ? (int64_t)((16u - mis) / ES) : 0;
  if (h > n) h = n;
  const int64_t nb = (n - h) / VE;
  const int64_t tail0 = h + nb * VE;
  constexpr int64_t chunk = (int64_t)kScaleThreads * kScaleSlots;
  const uint32_t voff = threadIdx.x * 16u;
  for (int64_t v0 = (int64_t)blockIdx.x * chunk; v0 < nb; v0 += (int64_t)gridDim.x * chunk) {
    const int64_t cnt = nb - v0 < chunk ? nb - v0 : chunk;
    const rsrc_t r = make_rsrc(g + h + v0 * VE, (uint32_t)(cnt * 16));
    u32x4 v[kScaleSlots];
#pragma unroll
    for (int k = 0; k < kScaleSlots; ++k)
      v[k] = bload128<kPolicyStream>(r, voff, (uint32_t)k * kScaleThreads * 16u);
#pragma unroll
    for (int k = 0; k < kScaleSlots; ++k) {
      float f[VE];
      E::unpack(v[k], f);
#pragma unroll
      for (int i = 0; i < VE; ++i) f[i] *= sc;
      bstore128<kPolicyStream>(E::pack(f), r, voff, (uint32_t)k * kScaleThreads * 16u);
    }
  }
  if (blockIdx.x == 0) {
    const int64_t i = threadIdx.x;
    int64_t e = -1;
    if (i < h) e = i;
    else if (i - h < n - tail0) e = tail0 + (i - h);
    if (e >= 0) E::store1(g + e, E::load1(g + e) * sc);
  }
}

// ===========================================================================
// Streaming copy with the memory pattern of the row-part kernel (1024
// threads, 8 slots of 16-byte non-temporal loads issued before the stores,
// 128 KiB per workgroup): the achievable-bandwidth reference that the
// benchmark reports beside the cross-entropy kernel.  Not part of the
// method.
// ===========================================================================
constexpr int kCopyThreads = 1024;
constexpr int kCopySlots = 8;
constexpr int64_t kCopyChunk = (int64_t)kCopyThreads * kCopySlots * 16;

__global__ __launch_bounds__(kCopyThreads) void ce_copy_kernel(const char* __restrict__ src,
                                                               char* __restrict__ dst,
                                                               int64_t bytes) {
  const int64_t base = (int64_t)blockIdx.x * kCopyChunk;
  if (base >= bytes) return;
  const uint32_t n = (uint32_t)(bytes - base < kCopyChunk ? bytes - base : kCopyChunk);
  const rsrc_t ri = make_rsrc(src + base, n), ro = make_rsrc(dst + base, n);
  const uint32_t voff = threadIdx.x * 16u;
  u32x4 v[kCopySlots];
#pragma unroll
  for (int k = 0; k < kCopySlots; ++k)
    v[k] = bload128<kPolicyStream>(ri, voff, (uint32_t)k * kCopyThreads * 16u);
#pragma unroll
  for (int k = 0; k < kCopySlots; ++k) asm volatile("" : "+v"(v[k]));
#pragma unroll
  for (int k = 0; k < kCopySlots; ++k)
    bstore128<kPolicyStream>(v[k], ro, voff, (uint32_t)k * kCopyThreads * 16u);
}

}  // namespace ce
