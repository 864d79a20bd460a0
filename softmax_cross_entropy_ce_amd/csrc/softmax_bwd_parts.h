// Softmax backward on long rows cut into parts (rumus project page,
// milestone M8c: the softmax backward kernel; dx = y (dy - <dy, y>)).
//
// A row of 128256 bf16 values holds 2 x 250 KB of y and dy; one workgroup
// cannot keep both on chip with more than one row in flight per CU.  Here
// the row's body (16-byte vectors from its first 128-byte boundary) is cut
// into P parts, one 1024-thread workgroup each, two workgroups per CU (at
// most 64 VGPRs).  A part loads its vectors of y and dy into NR register
// slots each, reduces its partial dot d_p = sum y dy in a fixed order, and
// trades d_p with the other parts; every part then adds the P partials in
// part order (d_0 first) and writes its share of dx from registers.
//
// The trade follows the row-part protocol of the cross-entropy kernel
// (ce_parts.h), with one float per part instead of a (max, sum) pair:
//  - part p's mailbox is P 64-bit words at the start of its own last two
//    body vectors in dx (four for eight parts); word q receives d_q as
//    [kMailTag | bits(d_q)];
//  - first thing, p sets its words to the empty tag; partners publish with
//    compare-and-swap from the empty tag, repeat the publish on every
//    fourth poll of their own mailbox while partials are missing (eight
//    parts also once more when the last one arrives, if a poll has skipped
//    its publish since the one before), and never wait for a publish's
//    result;
//  - p polls a bounded number of times; a partial that has not arrived by
//    then is recomputed from y and dy with the same slots, order and
//    workgroup reduction as its part uses, so the bits do not depend on
//    timing;
//  - both tags are signalling NaNs (as float32 and as 16-bit pairs), which
//    no arithmetic result is, so dx values never look like mailbox words.
// dx must not overlap y or dy (a recompute reads a partner's y and dy).
#pragma once

#include "ce_parts.h"

namespace ce {

// Sum over the workgroup in a fixed order: the wave's DPP reduction, then
// the waves' sums through LDS added in wave order by every wave.  Contains
// one barrier; the caller separates two uses by another.
template <int NW>
__device__ __forceinline__ float wg_sum(float v, float* red, int lane, int wv) {
  const float w = wave_allreduce(v, OpAdd{});
  if (lane == 0) red[wv] = w;
  __syncthreads();
  const float x = lane < NW ? red[lane] : 0.f;
  return wave_uniform(seg_allreduce<16>(x, OpAdd{}));
}

template <typename T, int P, int NT, int NR>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8)))
void sm_bwd_part_kernel(const T* __restrict__ y, const T* __restrict__ dy, int64_t B, int C,
                        T* __restrict__ dx, int spin, uint32_t* __restrict__ fallbacks) {
  using E = Elem<T>;
  constexpr int NW = NT / 64, VE = E::VE;
  static_assert(P == 2 || P == 4 || P == 8, "two, four or eight parts per row");
  // mailbox vectors at the end of each part: P 64-bit words
  constexpr int MV = P <= 4 ? 2 : P / 2;
  // eight parts keep the loops over partners rolled (less code, and no
  // partner's address held beyond its iteration: the kernel is capped at
  // 64 VGPRs)
  constexpr int kUnrollPartners = P <= 4 ? P : 1;
  static_assert(NT % 64 == 0 && NW >= 1 && NW <= 16, "1 to 16 waves");
  __shared__ float red[NW];
  __shared__ float mail[P];
  __shared__ int got[P];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t voff = (uint32_t)tid * 16u;
  int64_t row;
  int part;
  part_of_block<P>(blockIdx.x, row, part);
  if (row >= B) return;  // whole workgroup (and every part of the row)

  const T* yp = y + row * C;
  const T* dp = dy + row * C;
  T* op = dx + row * C;
  const RowGeom geo = row_geom<T, kPartAlign>(yp, C);
  const PartRange own = part_range(geo.nb, P, part);
  auto rsrc_of = [&](const T* base, const PartRange& pr) {
    return make_rsrc(base + geo.h + (int64_t)pr.v0 * VE, (uint32_t)pr.len * 16u);
  };
  const rsrc_t ry = rsrc_of(yp, own), rd = rsrc_of(dp, own);
  const rsrc_t ro = make_rsrc(op + geo.h + (int64_t)own.v0 * VE, (uint32_t)own.len * 16u);

  // every load of this part (lanes past its end read zeros)
  u32x4 vy[NR], vd[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    vy[k] = bload128<kPolicyStream>(ry, voff, (uint32_t)k * NT * 16u);
    vd[k] = bload128<kPolicyStream>(rd, voff, (uint32_t)k * NT * 16u);
  }
  // this part's mailbox: P words at the start of its last MV body vectors
  auto mailbox = [&](const PartRange& pr) {
    return reinterpret_cast<uint64_t*>(op + geo.h + (int64_t)(pr.v0 + pr.len - MV) * VE);
  };
  uint64_t* const mine = mailbox(own);
  constexpr uint64_t kEmptyWord = (uint64_t)kMailEmpty << 32;
  if (tid == 0) {
#pragma unroll
    for (int q = 0; q < P; ++q)
      __hip_atomic_store(&mine[q], kEmptyWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // edge elements of part q: the head belongs to part 0, the tail to part
  // P-1; edge i goes to thread i
  auto edge_elem = [&](int q) -> int {
    const int nh = q == 0 ? geo.h : 0;
    const int nt = q == P - 1 ? geo.ntail : 0;
    if (tid < nh) return tid;
    if (tid - nh < nt) return geo.tail0 + (tid - nh);
    return -1;
  };
  const int xe = edge_elem(part);
  const float ey = xe >= 0 ? E::load1(yp + xe) : 0.f;
  const float ed = xe >= 0 ? E::load1(dp + xe) : 0.f;

  // a part's partial dot: its slots in order, then its edge element (the
  // recompute below adds the same terms in the same order)
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < NR; ++k)
    if (k * NT < own.len) acc += vec_dot<T>(vy[k], vd[k]);
  // the edge term in the same form as in the recompute (a product chosen
  // against 0, then one add), so both round alike
  const float e_own = xe >= 0 ? ey * ed : 0.f;
  const float d_own = wg_sum<NW>(acc + e_own, red, lane, wv);

  // trade the partials
  if (tid < P) got[tid] = tid == part ? 1 : 0;
  if (tid == 0) {
    mail[part] = d_own;
    const uint64_t word = ((uint64_t)kMailTag << 32) | __builtin_bit_cast(uint32_t, d_own);
    auto publish = [&] {
#pragma unroll kUnrollPartners
      for (int q = 0; q < P; ++q) {
        if (q == part) continue;
        uint64_t e = kEmptyWord;
        __hip_atomic_compare_exchange_strong(&mailbox(part_range(geo.nb, P, q))[part], &e, word,
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        wide_store_guard();  // 16 bytes of data, as a wide store
      }
    };
    publish();
    int have = 1;
    bool behind = false;  // a pass has skipped its publish since the last one
    for (int it = 0; it < spin && have < P; ++it) {
#pragma unroll kUnrollPartners
      for (int q = 0; q < P; ++q) {
        if (q == part || got[q]) continue;
        const uint64_t w = __hip_atomic_load(&mine[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) == kMailTag) {
          mail[q] = __builtin_bit_cast(float, (uint32_t)w);
          got[q] = 1;
          ++have;
        }
      }
      const bool done = have == P;
      if (done ? (P == 8 && behind) : (it & 3) == 3) {
        publish();
        behind = false;
      } else {
        behind = !done;
      }
      if (!done) __builtin_amdgcn_s_sleep(8);
    }
    if (fallbacks != nullptr && have < P) atomicAdd(fallbacks, (uint32_t)(P - have));
  }
  __syncthreads();
  // recompute what did not arrive, with the part's own slots and order
#pragma unroll kUnrollPartners
  for (int q = 0; q < P; ++q) {
    if (got[q]) continue;  // uniform (LDS, after the barrier)
    const PartRange pq = part_range(geo.nb, P, q);
    const rsrc_t qy = rsrc_of(yp, pq), qd = rsrc_of(dp, pq);
    // one slot at a time: this part's registers stay live for its dx
    float aq = 0.f;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      if (k * NT >= pq.len) break;  // uniform
      const u32x4 a = bload128<kPolicyStream>(qy, voff, (uint32_t)k * NT * 16u);
      const u32x4 b = bload128<kPolicyStream>(qd, voff, (uint32_t)k * NT * 16u);
      aq += vec_dot<T>(a, b);
    }
    const int xq = edge_elem(q);
    const float eq = xq >= 0 ? E::load1(yp + xq) * E::load1(dp + xq) : 0.f;
    const float dq = wg_sum<NW>(aq + eq, red, lane, wv);
    __syncthreads();  // red is reused by the next recompute
    if (tid == 0) mail[q] = dq;
  }
  __syncthreads();
  float dot = 0.f;
#pragma unroll
  for (int q = 0; q < P; ++q) dot = dot + mail[q];

  // dx of this part from the registers, over the mailbox too
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    asm volatile("" : "+v"(vy[k]));
    asm volatile("" : "+v"(vd[k]));
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    if (k * NT >= own.len) break;  // uniform
    bstore128<kPolicyStream>(vec_dx<T>(vy[k], vd[k], dot), ro, voff, (uint32_t)k * NT * 16u);
  }
  if (xe >= 0) E::store1(op + xe, ey * (ed - dot));
}

}  // namespace ce
