// Path 4: rows cut into parts, one workgroup per part and several
// workgroups per CU.
//
// The method's per-row steps (rumus 0.1.1 cross_entropy.wgsl, pass 1 steps
// 1-4 and pass 2) need the row's max and sum of exponentials before any
// gradient element can be written.  With one workgroup per row, a row of
// 128256 bf16 values (256 KB) fills a CU's registers and LDS, so only one
// row is in flight per CU.  Here a row of nb 16-byte vectors is cut into P
// parts.  A part is read once into registers (NR slots of NT vectors) and
// LDS (NL slots of NT vectors, then a partial slot of NXW waves), so that
// two or three workgroups of at most 64 VGPRs fill a CU's 32 wave slots
// and its LDS.  Each part is reduced to its own online
// (c, s) pair, and the parts then trade their pairs, so that every part
// combines the same P pairs in the same order (part 0 first) and writes
// its share of the gradient from on-chip data.  The combine is the
// online-softmax merge of (max, sum) partials.
//
// Trading pairs between workgroups.  Each part has a mailbox in grad: a
// pair of 64-bit words for each other part of its row, at the start of its
// own last P - 1 body vectors.  Every other part publishes its (c, s) into
// its pair of words, one value per word in the low half with kMailTag in
// the high half; the owner polls them, and its own gradient store
// overwrites them only after the poll has ended.
//  - First thing, the owner sets its words to kMailEmpty.  Its own later
//    polls are ordered after that store, so whatever grad held before the
//    call can never be read as a partner's value.
//  - The partner publishes with compare-and-swap from kMailEmpty, so a
//    publish that meets anything else (data from before the owner's
//    emptying, or the owner's gradient once the owner has given up) changes
//    nothing.  It repeats the publish on every poll of its own mailbox, so
//    a publish that an owner starting late has emptied again is made
//    again.  (One more publish after the partner's own pair has arrived
//    was measured to cost about 1 % and is not made: the rare publish it
//    would save ends in the recompute below.)
//  - Both tags are signalling NaNs, both as one float32 and as two bf16
//    values.  No arithmetic result is a signalling NaN, so no gradient
//    value can look like a mailbox word, and a word with kMailTag that the
//    owner reads was written by the partner in this launch.
//  - The owner polls a bounded number of times.  If the pair has not come
//    by then (the partner is not resident yet, or its publish was erased),
//    it recomputes the pair from the logits with the same code, slots and
//    order that the partner uses.  The result is bitwise the same whichever
//    way the pair arrived.  No wait is unbounded and no result depends on
//    timing.
//
// Workgroup g runs on XCD g % 8 (round-robin dispatch); the parts of a row
// are given workgroups g, g + 8, ..., so they share an XCD and start next to
// each other in its dispatch order.  Rows are cut into one, two, four or
// eight parts.
#pragma once

#include "ce_kernels.h"

namespace ce {

constexpr uint32_t kMailTag = 0x7FA57FA5u;
constexpr uint32_t kMailEmpty = 0x7FA17FA1u;

// A part's body starts at a 128-byte boundary of the logits row (one cache
// line), and parts are whole multiples of 8 vectors, so every wave's 1 KB
// access covers whole lines; the up to 128/size - 1 elements before the
// boundary are head elements handled one per thread.
constexpr int kPartAlign = 128;
constexpr int kPartQuantum = kPartAlign / 16;

// Body-vector range [v0, v0 + len) of part q when nb vectors are cut into P
// parts of ceil(nb / P) rounded up to whole cache lines.
struct PartRange {
  int v0, len;
};
__device__ __forceinline__ PartRange part_range(int nb, int P, int q) {
  const int L = ((nb + P - 1) / P + kPartQuantum - 1) / kPartQuantum * kPartQuantum;
  const int a = q * L < nb ? q * L : nb;
  const int b = a + L < nb ? a + L : nb;
  return PartRange{a, b - a};
}

// Workgroup index -> (row, part): parts of one row on one XCD, consecutive
// in its dispatch order.
template <int P>
__device__ __forceinline__ void part_of_block(uint32_t g, int64_t& row, int& part) {
  const uint32_t xcd = g & 7u, local = g >> 3;
  row = (int64_t)(local / P) * 8 + xcd;
  part = (int)(local % P);
}

// Max / sum pair of the whole workgroup, from each thread's (c, s).  Every
// thread gets the same result; the order of operations is fixed.  Contains
// one barrier; the caller separates two uses by another.
template <int NW>
__device__ __forceinline__ void wg_pair(float c, float s, float* red_c, float* red_s, int lane,
                                        int wv, float& cg, float& sg) {
  const float cw = wave_allreduce(c, OpMax{});
  const float sw = wave_allreduce(s * exp2_hw(c - cw), OpAdd{});
  if (lane == 0) {
    red_c[wv] = cw;
    red_s[wv] = sw;
  }
  __syncthreads();
  const float ci = lane < NW ? red_c[lane] : kLowest;
  const float si = lane < NW ? red_s[lane] : 0.f;
  cg = wave_uniform(seg_allreduce<16>(ci, OpMax{}));
  sg = wave_uniform(seg_allreduce<16>(si * exp2_hw(ci - cg), OpAdd{}));
}

// Vectors a part of ce_part_kernel<T, P, NT, NR, NL, NXW> holds.
constexpr int part_capacity(int NT, int NR, int NL, int NXW) { return (NR + NL) * NT + NXW * 64; }

// fallbacks (may be null): a device counter, incremented once by every part
// that recomputed its partner's pair instead of receiving it.  spin: polls
// before that happens (0: every part recomputes).  At most 64 VGPRs (eight
// waves per SIMD), so 32 / (NT / 64) workgroups fit a CU by waves.
template <typename T, int P, int NT, int NR, int NL, int NXW, int OP = kOpCE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8)))
void ce_part_kernel(const T* __restrict__ logits, const int32_t* __restrict__ targets, int64_t B,
                    int C, RowArgs rs, T* __restrict__ grad, float* __restrict__ loss_rows,
                    int spin, uint32_t* __restrict__ fallbacks) {
  const float invB = row_invB(rs), gmul = grad_mul(rs);
  using E = Elem<T>;
  constexpr int NW = NT / 64, VE = E::VE, ES = sizeof(T);
  constexpr int NLS = NL + (NXW > 0 ? 1 : 0);  // LDS slots, the last maybe partial
  constexpr int NS = NR + NLS;                 // slots per part
  constexpr int NX = NXW * 64;                 // threads with a vector in the partial slot
  static_assert(P == 1 || P == 2 || P == 4 || P == 8, "one, two, four or eight parts per row");
  static_assert(NT % 64 == 0 && NW >= 1 && NW <= 16, "1 to 16 waves");
  static_assert(NXW >= 0 && NXW < NW, "partial LDS slot smaller than a slot");
  __shared__ u32x4 stage[NL * NT + NX > 0 ? NL * NT + NX : 1];
  __shared__ float red_c[NW], red_s[NW];
  __shared__ float mail_c[P], mail_s[P];
  __shared__ int mail_ok[P];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t voff = (uint32_t)tid * 16u;
  int64_t row;
  int part;
  part_of_block<P>(blockIdx.x, row, part);
  if (row >= B) return;  // whole workgroup (and every part of the row)

  const T* rp = logits + row * rs.ldz;
  T* gp = grad + row * rs.ldg;
  const RowGeom geo = row_geom<T, kPartAlign>(rp, C);
  const PartRange own = part_range(geo.nb, P, part);
  const rsrc_t rrow = make_rsrc(rp, (uint32_t)C * ES);
  const rsrc_t rin = make_rsrc(rp + geo.h + own.v0 * VE, (uint32_t)own.len * 16u);
  const rsrc_t rout = make_rsrc(gp + geo.h + own.v0 * VE, (uint32_t)own.len * 16u);

  // Phase A: every load of this part, register slots first.
  u32x4 v[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) v[k] = bload128<kPolicyStream>(rin, voff, (uint32_t)k * NT * 16u);
#pragma unroll
  for (int p = 0; p < NL; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rin, (lds_ptr_t)&stage[p * NT + wv * 64], 16, voff,
                                             (uint32_t)(NR + p) * NT * 16u, 0, kPolicyStream);
  if constexpr (NXW > 0) {
    if (wv < NXW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rin, (lds_ptr_t)&stage[NL * NT + wv * 64], 16, voff,
                                               (uint32_t)(NR + NL) * NT * 16u, 0, kPolicyStream);
  }
  // Empty this part's mailbox (rows of several parts) before anything can
  // be published into it: P - 1 pairs of words, one pair per other part,
  // at the start of the part's last P - 1 body vectors.
  constexpr int NM = P - 1;
  auto mailbox = [&](const PartRange& pr) {
    return reinterpret_cast<uint64_t*>(gp + geo.h + (int64_t)(pr.v0 + pr.len - NM) * VE);
  };
  // the pair of words that part `from` publishes into part `to`'s mailbox
  auto mail_index = [](int from, int to) { return 2 * (from < to ? from : from - 1); };
  uint64_t* const mine = P > 1 ? mailbox(own) : nullptr;
  constexpr uint64_t kEmptyWord = (uint64_t)kMailEmpty << 32;
  if constexpr (P > 1) {
    if (tid == 0) {
#pragma unroll
      for (int w = 0; w < 2 * NM; ++w)
        __hip_atomic_store(&mine[w], kEmptyWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // LDS slot p of this thread (the partial slot holds nothing for threads
  // at or past NX: their vectors lie past every part's end).
  auto lds_slot = [&](int p) -> u32x4 {
    if (p < NL || tid < NX) return stage[p * NT + tid];
    return u32x4{0u, 0u, 0u, 0u};
  };

  static_assert(OP != kOpShard, "shard records come from the row kernels");
  const RowTarget rt = row_target<OP>(targets, row, C, rs);
  const int t = rt.t;
  const bool valid = rt.valid;
  const int tb = t >= 0 ? t - geo.h : -1;
  const bool t_body = tb >= 0 && tb < geo.nb * VE;
  const int tvec = t_body ? tb / VE : -1;  // target's body vector (row-relative)
  const int tj = t_body ? tb % VE : -1;

  // Edge elements of part q: the head (before the first 128-byte boundary)
  // belongs to part 0 and the tail to part P-1; edge i goes to thread i.
  auto edge_elem = [&](int q) -> int {
    const int nh = q == 0 ? geo.h : 0;
    const int nt = q == P - 1 ? geo.ntail : 0;
    if (tid < nh) return tid;
    if (tid - nh < nt) return geo.tail0 + (tid - nh);
    return -1;
  };
  const int xe = edge_elem(part);
  const float xs_raw = bload_elem<T>(rrow, (uint32_t)(xe >= 0 ? xe : C) * ES);
  const float zt_raw = bload_elem<T>(rrow, (uint32_t)(t >= 0 ? t : C) * ES);

  // The target element.  The thread whose vectors hold it sets it to -inf
  // in the loaded data, once, so no slot needs per-element target code; the
  // part folds z_t into its running max after its slots (the target stays
  // out of the sum), and the owning thread stores g_t after its vector
  // stores.  Per part q: whether this wave holds the target's vector, and
  // the slot that holds it for the owning thread (-1 for the others).
  struct TargetIn {
    bool wave;
    int k;
  };
  auto target_in = [&](const PartRange& pr) -> TargetIn {
    const bool in = t_body && tvec >= pr.v0 && tvec < pr.v0 + pr.len;
    const bool mine = in && (tvec - pr.v0) % NT == tid;
    return TargetIn{__builtin_amdgcn_ballot_w64(mine) != 0, mine ? (tvec - pr.v0) / NT : -1};
  };
  const TargetIn tin = target_in(own);

  // Slot k of part q (this thread's vector k*NT + tid of the part) as
  // floats.  Slots past the part's end are skipped as a whole (uniform);
  // lanes past it hold -inf.
  auto slot_values = [&](const PartRange& pr, const TargetIn& ti, int k, u32x4 w,
                         float (&f)[VE]) {
    if (ti.wave && ti.k == k) w = E::kill(w, tj);
    E::unpack(w, f);
    if (k * NT + NT > pr.len) {
      const bool ok = tid < pr.len - k * NT;
#pragma unroll
      for (int i = 0; i < VE; ++i) f[i] = ok ? f[i] : kNegInf;
    }
  };
  auto fold_slot = [&](const PartRange& pr, const TargetIn& ti, int k, u32x4 w, float& c,
                       float& s) {
    if (k * NT >= pr.len) return;
    float f[VE];
    slot_values(pr, ti, k, w, f);
    online_fold(c, s, max_of(f), f);
  };
  auto fold_edge = [&](int e, float x, float& c, float& s) {
    if (e >= 0) {
      const float one[1] = {(e == t) ? kNegInf : x};
      online_fold(c, s, x, one);
    }
  };
  // z_t into the running max of the part whose body holds it (max only)
  auto fold_target_max = [&](const PartRange& pr, float zt_, float& c, float& s) {
    if (t_body && tvec >= pr.v0 && tvec < pr.v0 + pr.len) {
      const float none[1] = {kNegInf};
      online_fold(c, s, zt_, none);
    }
  };

  // Phase B: this part's pair.  For fp32, the register slots keep each
  // element's term 2^(z log2e - c_k) in place of z, with c_k the running max
  // after slot k, so that the gradient needs one multiply per element.
  // Eight parts recompute the terms instead: the running maxima, with the
  // code that trades eight pairs, would not fit the 64 VGPRs.
  constexpr bool kKeepTerms = sizeof(T) == 4 && P <= 4;
  float ck[NR];
  float c = kLowest, s = 0.f;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    ck[k] = c;
    if (k * NT >= own.len) continue;
    float f[VE];
    slot_values(own, tin, k, v[k], f);
    if constexpr (kKeepTerms) {
      float e[VE];
      online_fold_e(c, s, max_of(f), f, e);
      ck[k] = c;
      v[k] = as_u32(f32x4{e[0], e[1], e[2], e[3]});
    } else {
      online_fold(c, s, max_of(f), f);
    }
  }
  wait_vmcnt<0>();  // LDS slots, edge and target loads
#pragma unroll
  for (int p = 0; p < NLS; ++p) fold_slot(own, tin, NR + p, lds_slot(p), c, s);
  const float xs = xe >= 0 ? xs_raw : kNegInf;
  const float zt = t >= 0 ? zt_raw : 0.f;
  fold_edge(xe, xs, c, s);
  fold_target_max(own, zt, c, s);
  float c_own, s_own;
  wg_pair<NW>(c, s, red_c, red_s, lane, wv, c_own, s_own);

  // The pairs of all parts, in LDS: this part's own, the others' as
  // received, or recomputed where a partner's did not arrive in time.
  float cg = c_own, sx = s_own;
  if constexpr (P > 1) {
    // Eight parts keep the loops over partners rolled (less code, and no
    // partner's address or pair held beyond its iteration: the kernel is
    // capped at 64 VGPRs).
    constexpr int kUnrollPartners = P <= 4 ? P : 1;
    if (tid == 0) {
      mail_c[part] = c_own;
      mail_s[part] = s_own;
      const uint64_t tag = (uint64_t)kMailTag << 32;
      const uint64_t w0 = tag | __builtin_bit_cast(uint32_t, c_own);
      const uint64_t w1 = tag | __builtin_bit_cast(uint32_t, s_own);
      // The publishes are issued without waiting for their results, so the
      // next poll follows them at once.
      auto publish = [&] {
#pragma unroll kUnrollPartners
        for (int q = 0; q < P; ++q) {
          if (q == part) continue;
          uint64_t* m = mailbox(part_range(geo.nb, P, q)) + mail_index(part, q);
          uint64_t e0 = kEmptyWord, e1 = kEmptyWord;
          // a 64-bit compare-and-swap sends 16 bytes of data: the same
          // wait states as a wide store follow it
          __hip_atomic_compare_exchange_strong(&m[0], &e0, w0, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          wide_store_guard();
          __hip_atomic_compare_exchange_strong(&m[1], &e1, w1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          wide_store_guard();
        }
      };
      publish();
      // a bit per part whose pair is here; received pairs go straight to LDS
      constexpr unsigned kAll = (1u << P) - 1u;
      unsigned got = 1u << part;
      for (int it = 0; it < spin && got != kAll; ++it) {
#pragma unroll kUnrollPartners
        for (int q = 0; q < P; ++q) {
          if ((got >> q) & 1u) continue;
          const uint64_t* m = mine + mail_index(q, part);
          const uint64_t a = __hip_atomic_load(&m[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t b = __hip_atomic_load(&m[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((uint32_t)(a >> 32) == kMailTag && (uint32_t)(b >> 32) == kMailTag) {
            mail_c[q] = __builtin_bit_cast(float, (uint32_t)a);
            mail_s[q] = __builtin_bit_cast(float, (uint32_t)b);
            got |= 1u << q;
          }
        }
        if (got != kAll) {
          publish();
          __builtin_amdgcn_s_sleep(8);
        }
      }
#pragma unroll
      for (int q = 0; q < P; ++q) mail_ok[q] = (int)((got >> q) & 1u);
      if (got != kAll && fallbacks != nullptr)
        atomicAdd(fallbacks, (uint32_t)(P - __builtin_popcount(got)));
    }
    __syncthreads();
#pragma unroll kUnrollPartners
    for (int q = 0; q < P; ++q) {
      if (q == part || mail_ok[q]) continue;  // uniform (LDS, after the barrier)
      // Recompute part q's pair: the same slots, fold order, edges and
      // workgroup reduction as part q runs itself.
      const PartRange pq = part_range(geo.nb, P, q);
      const rsrc_t rq = make_rsrc(rp + geo.h + pq.v0 * VE, (uint32_t)pq.len * 16u);
      const TargetIn tq = target_in(pq);
      float cq = kLowest, sq = 0.f;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const u32x4 w = bload128<kPolicyStream>(rq, voff, (uint32_t)k * NT * 16u);
        fold_slot(pq, tq, k, w, cq, sq);
      }
      const int xq = edge_elem(q);
      const float xqv = bload_elem<T>(rrow, (uint32_t)(xq >= 0 ? xq : C) * ES);
      fold_edge(xq, xq >= 0 ? xqv : kNegInf, cq, sq);
      fold_target_max(pq, zt, cq, sq);
      float cr, sr;
      wg_pair<NW>(cq, sq, red_c, red_s, lane, wv, cr, sr);
      if (tid == 0) {
        mail_c[q] = cr;
        mail_s[q] = sr;
      }
      __syncthreads();  // the pair is in LDS; red_c / red_s may be used again
    }
    // Combine the parts' pairs in part order.
    cg = mail_c[0];
#pragma unroll
    for (int q = 1; q < P; ++q) cg = __builtin_fmaxf(cg, mail_c[q]);
    // the maxima are read from LDS again rather than kept in registers
    if constexpr (P > 4) asm volatile("" ::: "memory");
    sx = mail_s[0] * exp2_hw(mail_c[0] - cg);
#pragma unroll
    for (int q = 1; q < P; ++q) sx = sx + mail_s[q] * exp2_hw(mail_c[q] - cg);
  }
  const RowResult rr = row_finish<OP>(cg, sx, zt, valid, rt.ignored, invB, gmul);
  if (part == 0 && tid == 0) store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);

  // Phase C: the gradient of this part from registers and LDS.
  auto write_slot = [&](int k, u32x4 w) {
    if (k * NT >= own.len) return;
    float f[VE], g[VE];
    E::unpack(w, f);
#pragma unroll
    for (int i = 0; i < VE; ++i) g[i] = exp2_hw(__builtin_fmaf(f[i], kLog2e, -cg)) * rr.scale;
    bstore128<kPolicyStream>(E::pack(g), rout, voff, (uint32_t)k * NT * 16u);
  };
#pragma unroll
  for (int k = 0; k < NR; ++k) asm volatile("" : "+v"(v[k]));
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    if constexpr (kKeepTerms) {
      if (k * NT >= own.len) continue;
      const float factor = exp2_hw(ck[k] - cg) * rr.scale;
      const f32x4 e = as_f32(v[k]);
      const f32x4 g = {e.x * factor, e.y * factor, e.z * factor, e.w * factor};
      bstore128<kPolicyStream>(as_u32(g), rout, voff, (uint32_t)k * NT * 16u);
    } else {
      write_slot(k, v[k]);
    }
  }
#pragma unroll
  for (int p = 0; p < NLS; ++p) {
    if (p < NL || tid < NX) write_slot(NR + p, lds_slot(p));
  }
  if (xe >= 0) {
    const float g = (xe == t) ? rr.gt : exp2_hw(__builtin_fmaf(xs, kLog2e, -cg)) * rr.scale;
    E::store1(gp + xe, g);
  }
  // the target's gradient, over the value its vector store wrote there (the
  // same thread, the same address, later in program order)
  if (tin.k >= 0) E::store1(gp + geo.h + (int64_t)tvec * VE + tj, rr.gt);
}

}  // namespace ce
