// Cross-entropy over a vocabulary split into column shards.
//
// An LM head split along its output features (rumus project page, milestone
// M24: a column-parallel linear layer) leaves each rank the logits of a
// contiguous range of classes.  The cross-entropy of the whole row then
// takes two passes over a shard, with one exchange between them:
//   1. every shard reduces each row to a record (the row kernels with
//      kOpShard: c, sx, zt, own; one read of the shard);
//   2. the records of all shards are gathered (on several GPUs an
//      all-gather of B x 16 bytes per shard; here the caller stacks them);
//   3. every shard combines the records of a row in shard order and writes
//      its columns of the gradient (this kernel: one more read of the shard
//      and one write).
// The combine is the merge of (max, sum) partials that the row-part kernel
// applies to its parts: c = max_k c_k, sx = sum_k sx_k 2^(c_k - c) in shard
// order, zt from the shard that holds the target; row_epilogue then gives
// the loss, the gradient scale and the target's gradient.  Every shard does
// the same arithmetic on the same records, so all shards agree bit for bit
// on each row's values, whichever shard computes them.
#pragma once

#include "ce_kernels.h"

namespace ce {

// The combine of a row's records, shard by shard in shard order: every
// kernel below runs exactly this code, so all shards of a row, whichever
// kernel serves them, compute the same bits.
struct ShardRow {
  float c, sx, zt, own;
};
__device__ __forceinline__ ShardRow shard_combine(const f32x4* __restrict__ recs, int nshards,
                                                  int64_t B, int64_t row) {
  ShardRow r{kLowest, 0.f, 0.f, 0.f};
  for (int k = 0; k < nshards; ++k) r.c = fmax2(r.c, recs[(int64_t)k * B + row].x);
  for (int k = 0; k < nshards; ++k) {
    const f32x4 q = recs[(int64_t)k * B + row];
    r.sx = r.sx + q.y * exp2_hw(q.x - r.c);
    r.zt = r.zt + q.z;
    r.own = r.own + q.w;
  }
  return r;
}

// A unit of work is U threads x S slots: U * S body vectors of one row.
// Rows of at most 512 vectors take one wave x 8 slots; longer rows 256
// threads x 2 slots (512 vectors, several units per row), which measured
// 4-10 % faster than 256 x 8 on 8192 x 16032 and 8192 x 32064 bf16 and
// 4096 x 6282 fp32 shards (at a copy's rate on the last two).  1024 / U
// units share a 1024-thread workgroup (large workgroups stream faster than
// small ones on this GPU); they need no barrier, since every thread
// combines the records of its row by itself.
constexpr int kShardThreads = 1024;
constexpr int kShardTinyC = 16;                             // rows one thread handles

// Unit u (= 1024/U * workgroup + threadIdx.x / U) handles body vectors
// [j * U * 8, (j + 1) * U * 8) of row u / chunks (j = u % chunks), and
// chunk 0 also the row's elements before its first 16-byte boundary and
// after its last; units past B * chunks do nothing.  recs holds nshards x B
// records, shard-major.  A row whose target lies outside [0, Ctot), or is
// held by other than exactly one shard's record, gets NaN loss and
// gradient.
template <typename T, int U, int S>
__global__ __launch_bounds__(kShardThreads) void ce_shard_grad_kernel(
    const T* __restrict__ logits, const int32_t* __restrict__ targets, int64_t B, int C,
    int64_t col0, int64_t Ctot, const f32x4* __restrict__ recs, int nshards, RowArgs rs,
    T* __restrict__ grad, float* __restrict__ loss_rows, int chunks) {
  static_assert(U == 64 || U == 256, "a unit is one or four waves");
  constexpr int kUnits = kShardThreads / U;
  constexpr int kChunk = U * S;
  using E = Elem<T>;
  constexpr int VE = E::VE, NT = U;
  // wave-uniform (a unit is whole waves): readfirstlane lets the compiler
  // load the row's records and target with scalar loads
  const int64_t unit = (int64_t)blockIdx.x * kUnits +
                       __builtin_amdgcn_readfirstlane((int)(threadIdx.x / U));
  const int64_t row = unit / chunks;
  if (row >= B) return;  // whole waves
  const int chunk = (int)(unit % chunks);
  const int tid = threadIdx.x % U;
  const uint32_t voff = (uint32_t)tid * 16u;

  const T* rp = logits + row * rs.ldz;
  T* gp = grad + row * rs.ldg;
  const RowGeom geo = row_geom(rp, C);
  const int v0 = chunk * kChunk;
  const int nv = geo.nb - v0 < kChunk ? geo.nb - v0 : kChunk;
  const uint32_t bytes = nv > 0 ? (uint32_t)nv * 16u : 0u;
  const rsrc_t rin = make_rsrc(rp + geo.h + (int64_t)v0 * VE, bytes);
  const rsrc_t rout = make_rsrc(gp + geo.h + (int64_t)v0 * VE, bytes);
  u32x4 v[S];
#pragma unroll
  for (int k = 0; k < S; ++k)
    v[k] = bload128<kPolicyStream>(rin, voff, (uint32_t)k * NT * 16u);
  int xe = -1;  // chunk 0: this thread's edge element, if any
  if (chunk == 0) {
    if (tid < geo.h)
      xe = tid;
    else if (tid - geo.h < geo.ntail)
      xe = geo.tail0 + (tid - geo.h);
  }
  const float xs = xe >= 0 ? E::load1(rp + xe) : 0.f;

  const ShardRow sr = shard_combine(recs, nshards, B, row);
  const float c = sr.c;
  const int64_t tg = targets[row];
  const bool valid = tg >= 0 && tg < Ctot && sr.own == 1.f;
  const RowResult rr = row_epilogue(c, sr.sx, sr.zt, valid, rs.invB, grad_mul(rs));
  if (loss_rows != nullptr && chunk == 0 && tid == 0) loss_rows[row] = row_loss(rr);

  // the target's column in this shard, if it is here: body vector tvec
  // (element tj) or an edge element
  const int64_t tl = tg - col0;
  const int t = (tl >= 0 && tl < C) ? (int)tl : -1;
  const int tb = t - geo.h;
  const bool t_body = t >= 0 && tb >= 0 && tb < geo.nb * VE;
  const int tvec = t_body ? tb / VE - v0 : -1;  // chunk-relative
  const int tk = (tvec >= 0 && tvec < nv && tvec % NT == tid) ? tvec / NT : -1;
  const int tj = t_body ? tb % VE : 0;

#pragma unroll
  for (int k = 0; k < S; ++k) {
    if (k * NT >= nv) break;  // uniform
    float f[VE], g[VE];
    E::unpack(v[k], f);
#pragma unroll
    for (int i = 0; i < VE; ++i) g[i] = exp2_hw(__builtin_fmaf(f[i], kLog2e, -c)) * rr.scale;
    if (k == tk) {
#pragma unroll
      for (int i = 0; i < VE; ++i) g[i] = (i == tj) ? rr.gt : g[i];
    }
    bstore128<kPolicyStream>(E::pack(g), rout, voff, (uint32_t)k * NT * 16u);
  }
  if (xe >= 0) {
    const float g = (xe == t) ? rr.gt : exp2_hw(__builtin_fmaf(xs, kLog2e, -c)) * rr.scale;
    E::store1(gp + xe, g);
  }
}

// Shards of at most kShardTinyC columns (a vocabulary cut into more shards
// than it has many columns): one thread per row, elements loaded and stored
// one by one.  The records of a row then outweigh its elements, and a unit
// of whole waves per row would leave almost every lane idle.
template <typename T>
__global__ __launch_bounds__(256) void ce_shard_grad_tiny_kernel(
    const T* __restrict__ logits, const int32_t* __restrict__ targets, int64_t B, int C,
    int64_t col0, int64_t Ctot, const f32x4* __restrict__ recs, int nshards, RowArgs rs,
    T* __restrict__ grad, float* __restrict__ loss_rows) {
  using E = Elem<T>;
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= B) return;  // no barrier follows
  const ShardRow sr = shard_combine(recs, nshards, B, row);
  const int64_t tg = targets[row];
  const bool valid = tg >= 0 && tg < Ctot && sr.own == 1.f;
  const RowResult rr = row_epilogue(sr.c, sr.sx, sr.zt, valid, rs.invB, grad_mul(rs));
  if (loss_rows != nullptr) loss_rows[row] = row_loss(rr);
  const T* rp = logits + row * rs.ldz;
  T* gp = grad + row * rs.ldg;
  const int64_t tl = tg - col0;
  for (int j = 0; j < C; ++j) {
    const float x = E::load1(rp + j);
    const float g = j == tl ? rr.gt : exp2_hw(__builtin_fmaf(x, kLog2e, -sr.c)) * rr.scale;
    E::store1(gp + j, g);
  }
}

}  // namespace ce
