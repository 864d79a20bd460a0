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
//    nothing.  It repeats the publish on every fourth poll of its own
//    mailbox while pairs are missing, so that a publish that an owner
//    starting late has emptied again is made again.  (Every poll sent
//    2 P - 2 compare-and-swaps per waiting part; every fourth measured
//    0.7-1.8 points of 8 TB/s faster on rows of two, four and eight parts.)
//    Rows of eight parts publish once more when the last pair arrives, if
//    a poll has skipped its publish since the one before: without it a
//    few dozen parts a launch recomputed a pair.  (For fewer parts that
//    publish was measured to cost about 1 % and is not made: the rare
//    publish it would save ends in the recompute below.)
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
// each other in its dispatch order, and each XCD takes a contiguous block of
// rows (part_of_block_rows; rows of one part, and rows of eight parts in
// place, are dealt to the XCDs in turn).  Rows are cut into one, two, four
// or eight parts.
#pragma once

#include <type_traits>

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
// in its dispatch order; rows dealt to the XCDs in turn (row r on XCD
// r mod 8).
template <int P>
__device__ __forceinline__ void part_of_block(uint32_t g, int64_t& row, int& part) {
  const uint32_t xcd = g & 7u, local = g >> 3;
  row = (int64_t)(local / P) * 8 + xcd;
  part = (int)(local % P);
}

// The same for B rows with each XCD a contiguous block of ceil(B / 8) rows,
// taken in order: the cross-entropy rows of two or more parts.  (Rows dealt
// in turn measured slower there, fraction of 8 TB/s: 4096 x 50257 fp32
// 0.745 against 0.761, bf16 4096 x 151936 0.707 against 0.739, 16384 x
// 65536 0.691 against 0.738; 8192 x 128256 bf16 the same, 0.761.  Rows of
// one part measured the other way, e.g. bf16 65536 x 8192 0.787 dealt in
// turn against 0.717 in blocks and fp32 89472 x 3000 0.768 against 0.716,
// and so did rows of eight parts in place (bf16 2048 x 500000 0.695 against
// 0.658, fp32 2048 x 200000 0.681 against 0.632) and the softmax backward's
// parts (0.767 against 0.755 on 8192 x 128256 bf16): these keep
// part_of_block.)
template <int P>
__device__ __forceinline__ void part_of_block_rows(uint32_t g, int64_t B, int64_t& row,
                                                   int& part) {
  const uint32_t xcd = g & 7u, local = g >> 3;
  row = (int64_t)xcd * ((B + 7) / 8) + local / P;
  part = (int)(local % P);
}

// Maximum over the 16 lanes of each row of a wave: four v_max_f32 steps
// with their DPP operand (the compiler forms a max from a separate DPP move
// and a v_maximum3_f32 per step).  Each step is preceded by the two wait
// states a DPP read needs after a VALU write of its source.  v_max_f32
// returns the other operand for a quiet NaN; the values reduced here are
// finite, -inf or NaN from NaN inputs, whose sums are NaN regardless.
__device__ __forceinline__ float row16_max(float v) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf"
      : "+v"(v));
  return v;
}

// The same over the whole wave; the result is wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmax2(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                     kSwizzleXor16)));
  const float lo = __builtin_bit_cast(float,
                                      __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float hi = __builtin_bit_cast(float,
                                      __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  return fmax2(lo, hi);
}

// Each wave's max / sum pair, from each thread's (c, s), into red_c /
// red_s[wv] (lane 0 writes).  The caller puts a barrier before the reads.
__device__ __forceinline__ void wave_pair_to_lds(float c, float s, float* red_c, float* red_s,
                                                 int lane, int wv) {
  const float cw = wave_max(c);
  const float sw = wave_allreduce(s * exp2_hw(c - cw), OpAdd{});
  if (lane == 0) {
    red_c[wv] = cw;
    red_s[wv] = sw;
  }
}

// The NW waves' pairs in LDS combined into one, in a fixed order, by the
// calling wave (every lane gets the result).
template <int NW>
__device__ __forceinline__ void lds_pairs_combine(const float* red_c, const float* red_s, int lane,
                                                  float& cg, float& sg) {
  static_assert(NW <= 16, "one row of 16 lanes holds the waves' pairs");
  const float ci = lane < NW ? red_c[lane] : kLowest;
  const float si = lane < NW ? red_s[lane] : 0.f;
  cg = wave_uniform(row16_max(ci));
  sg = wave_uniform(seg_allreduce<16>(si * exp2_hw(ci - cg), OpAdd{}));
}

// The P parts' pairs combined in part order: cg = max c_q, then
// sx = sum over q of s_q * 2^(c_q - cg) starting from part 0.
template <int P>
__device__ __forceinline__ void combine_pairs(const float* mail_c, const float* mail_s, float& cg,
                                              float& sx) {
  cg = mail_c[0];
#pragma unroll
  for (int q = 1; q < P; ++q) cg = fmax2(cg, mail_c[q]);
  // the maxima are read from LDS again rather than kept in registers
  if constexpr (P > 4) asm volatile("" ::: "memory");
  sx = mail_s[0] * exp2_hw(mail_c[0] - cg);
#pragma unroll
  for (int q = 1; q < P; ++q) sx = sx + mail_s[q] * exp2_hw(mail_c[q] - cg);
}

// Max / sum pair of the whole workgroup, from each thread's (c, s).  Every
// thread gets the same result; the order of operations is fixed.  Contains
// one barrier; the caller separates two uses by another.
template <int NW>
__device__ __forceinline__ void wg_pair(float c, float s, float* red_c, float* red_s, int lane,
                                        int wv, float& cg, float& sg) {
  wave_pair_to_lds(c, s, red_c, red_s, lane, wv);
  __syncthreads();
  lds_pairs_combine<NW>(red_c, red_s, lane, cg, sg);
}

// In place (IP): rows of several parts whose gradient overwrites the
// logits.  A part cannot keep a mailbox in its own logits, and a part that
// stops waiting cannot recompute a partner's pair from the partner's
// logits, which may already be gradient.  So each row has a block of
// kInPlaceRowWords 64-bit words in a workspace (zero on entry and again on
// exit); a pair is stored as the bitwise complement of (c bits, s bits),
// so that 0 means empty.  A part that gives up waiting always ends without
// writing anything, so its logits are still there for the part that then
// writes its gradient.
//
// Two parts, words 0 and 1:
//  - each part, with its pair, tries to claim word 0 by compare-and-swap
//    from 0.  The part that claims it is the first; the other reads the
//    first's pair from it.
//  - the second publishes its pair into word 1 by compare-and-swap from 0
//    and writes its own half.
//  - the first polls word 1 a bounded number of times.  If the pair is
//    there it writes its own half; if not, it claims word 1 with
//    kInPlaceDeferred and ends without writing anything.  The second then
//    finds word 1 taken, and writes both halves.
//  - whoever reads the words last (the first when it found the pair, the
//    second when the first deferred) sets both back to 0.
//
// Four or eight parts: pair words 0..P-1, flag words 8..8+P-1, an arrival
// count (word 16) and a departure count (word 17), 32-bit counters that
// wrap to 0 after P:
//  - each part publishes its pair in its own word (an exchange whose
//    result it waits for, so the word is written before anything after),
//    then counts its arrival.  The part that arrives last is the closer:
//    every other part has published, so the closer gathers all pairs
//    (polling for words still on their way), then claims each other
//    part's flag with kInPlaceChecked by compare-and-swap from 0; a flag
//    that holds kInPlaceDeferred instead makes that part's gradient the
//    closer's to write, besides its own.
//  - any other part polls for all the pairs a bounded number of times.
//    With all of them it writes its own part.  Without, it claims its own
//    flag with kInPlaceDeferred: if that succeeds it ends without writing
//    (the closer, still to come, will find the mark); if the flag already
//    holds kInPlaceChecked, the closer has published, so the pairs are all
//    on their way: it polls for them again and writes its own part.
//  - every part counts its departure once its last access to the words has
//    completed; the last to leave sets the pair and flag words back to 0.
// Wave 0 runs this with lane q looking after part q's pair word and flag,
// so that a pass over the pairs or the flags is one access per lane (lane 0
// publishes and counts).
// No wait depends on a workgroup that has not started, and no part reads
// logits that may have been overwritten.  Every gradient element is
// 2^(z log2e - c') with the row's c', whichever part writes it, so the
// bits do not depend on who writes.
constexpr int kInPlaceRowWords = 18;
constexpr int kInPlaceFlags = 8;      // word index of the first flag
constexpr int kInPlaceCounts = 16;    // word index of the arrival count
constexpr int kInPlaceLongPolls = 1 << 16;  // polls for pairs already on their way
constexpr uint64_t kInPlaceChecked = 1;
constexpr uint64_t kInPlaceDeferred = ~(((uint64_t)kMailTag << 32) | kMailTag);

__device__ __forceinline__ uint64_t in_place_word(float c, float s) {
  return ~(((uint64_t)__builtin_bit_cast(uint32_t, c) << 32) | __builtin_bit_cast(uint32_t, s));
}
__device__ __forceinline__ void in_place_pair(uint64_t w, float& c, float& s) {
  c = __builtin_bit_cast(float, (uint32_t)(~w >> 32));
  s = __builtin_bit_cast(float, (uint32_t)~w);
}

// Vectors a part of ce_part_kernel<T, P, NT, NR, NL, NXW> holds.
constexpr int part_capacity(int NT, int NR, int NL, int NXW) { return (NR + NL) * NT + NXW * 64; }

// Waves per SIMD of a part kernel: eight (64 VGPRs, 32 waves per CU) for
// up to eight register slots, four (128 VGPRs) for more.
constexpr int part_waves(int NR) { return NR > 8 ? 4 : 8; }

// Register slots whose fp32 terms a 16-bit part keeps in LDS: as many as
// fit the CU's 160 KB shared by the workgroups that its waves allow, less
// 2 KB each for the reductions (32 bytes per thread and slot).
constexpr int part_lds_terms(int NT, int NR, int ES, int NL, int NXW) {
  const int wgs = 4 * part_waves(NR) * 64 / NT;
  const int budget = 160 * 1024 / wgs - 2048;
  const int n = budget / (NT * 32);
  return (ES != 2 || NL != 0 || NXW != 0) ? 0 : (n < NR ? n : NR);
}

// The max / sum pair of a part, in two passes over the data it holds:
//  1. the thread's maximum over its elements (16-bit types on their bit
//     patterns, pk_max16, with no widening; fp32 with max3);
//  2. the sum of 2^(z log2e - c) over them, c = that maximum times log2 e,
//     one fma and one v_exp_f32 per element, one c for all of the thread's
//     slots (no rescaling between slots).
// A partner that recomputes the pair runs the same two passes over the
// same slots in the same order, so the bits agree whichever way a pair
// arrives.
//
// Gradient of 16-bit types (and of fp32 in eight parts): each element's
// g = 2^(z log2e - c') with c' = cg - log2(1 / (S B)), the row's scale
// folded into the exponent, so that an element costs an fma, an exp and
// half a conversion.  A known upstream factor other than 1 multiplies
// after the exponential (a power of two then commutes with the rounding).
// fp32 in up to four parts keeps each element's term in its register slot
// and multiplies it by 2^(c - cg) / (S B).
//
// fallbacks (may be null): a device counter, incremented once by every part
// that recomputed its partner's pair instead of receiving it.  spin: polls
// before that happens (0: every part recomputes).  At most 64 VGPRs (eight
// waves per SIMD), so 32 / (NT / 64) workgroups fit a CU by waves.
//
// IP: the gradient in place of the logits (in_place: the rows' word blocks,
// see kInPlaceRowWords).
template <typename T, int P, int NT, int NR, int NL, int NXW, int OP = kOpCE, bool IP = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(part_waves(NR))))
void ce_part_kernel(const T* logits, const int32_t* __restrict__ targets, int64_t B, int C,
                    RowArgs rs, T* grad, float* __restrict__ loss_rows, int spin,
                    uint32_t* __restrict__ fallbacks, uint64_t* __restrict__ in_place) {
  const float invB = row_invB(rs), gmul = grad_mul(rs);
  using E = Elem<T>;
  constexpr int NW = NT / 64, VE = E::VE, ES = sizeof(T);
  constexpr bool k16 = sizeof(T) == 2;
  constexpr int NLS = NL + (NXW > 0 ? 1 : 0);  // LDS slots, the last maybe partial
  constexpr int NX = NXW * 64;                 // threads with a vector in the partial slot
  static_assert(P == 1 || P == 2 || P == 4 || P == 8, "one, two, four or eight parts per row");
  static_assert(NT % 64 == 0 && NW >= 1 && NW <= 16, "1 to 16 waves");
  static_assert(NXW >= 0 && NXW < NW, "partial LDS slot smaller than a slot");
  static_assert(!IP || (P >= 2 && OP == kOpCE), "in place: several parts, the loss with a gradient");
  // 16-bit parts held in registers alone keep the fp32 terms of their first
  // kLdsTerms register slots in LDS (32 bytes per thread and slot: two
  // slots, 64 KB, for 1024 threads, so two workgroups still fit a CU), so
  // that the gradient of those slots is one multiply per element instead
  // of an fma and an exponential.
  constexpr int kLdsTerms = IP ? 0 : part_lds_terms(NT, NR, sizeof(T), NL, NXW);
  static_assert(kLdsTerms <= NR, "kept slots are register slots");
  __shared__ u32x4 stage[NL * NT + NX > 0 ? NL * NT + NX : 1];
  __shared__ f32x4 kept[kLdsTerms > 0 ? kLdsTerms * 2 * NT : 1];
  __shared__ float red_c[NW], red_s[NW];
  __shared__ float mail_c[P], mail_s[P];
  __shared__ int mail_ok[P];
  // The row's results, formed once by wave 0 when every partner's pair
  // arrived (fin_ok) and read by every thread: cg, sx, 1/(S B), gmul/(S B),
  // g_t.
  __shared__ float fin[5];
  __shared__ int fin_ok;
  // in place: ip_deferred, this part ends without writing (its partner
  // writes its gradient); ip_extra, a bit per other part whose gradient
  // this part writes besides its own
  __shared__ int ip_deferred;
  __shared__ unsigned ip_extra;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t voff = (uint32_t)tid * 16u;
  int64_t row;
  int part;
  if constexpr (P == 1 || (IP && P == 8))
    part_of_block<P>(blockIdx.x, row, part);
  else
    part_of_block_rows<P>(blockIdx.x, B, row, part);
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
  if constexpr (P > 1 && !IP) {
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
  // in the loaded data, once, so no slot needs per-element target code; z_t
  // enters the maximum of the part whose body holds it (the target stays
  // out of the sum), and the owning thread stores g_t after its vector
  // stores.  Per part q: whether this wave holds the target's vector, and
  // the slot that holds it for the owning thread (-1 for the others).
  struct TargetIn {
    bool wave;  // this wave holds the target's vector
    int slot;   // the slot that holds it (the same for every thread), or -1
    bool mine;  // this thread holds it
    int k;      // slot for the owning thread, -1 for the others
    bool part;  // the part's body holds the target
  };
  auto target_in = [&](const PartRange& pr) -> TargetIn {
    const bool in = t_body && tvec >= pr.v0 && tvec < pr.v0 + pr.len;
    const bool mine = in && (tvec - pr.v0) % NT == tid;
    const int slot = in ? (tvec - pr.v0) / NT : -1;
    return TargetIn{__builtin_amdgcn_ballot_w64(mine) != 0, slot, mine, mine ? slot : -1, in};
  };
  const TargetIn tin = target_in(own);

  // Slot k of part q as it enters the pair: the target killed, lanes past
  // the part's end (last slot only; uniform test) set to -inf.  Slots wholly
  // past the end are skipped (uniform).
  auto slot_words = [&](const PartRange& pr, const TargetIn& ti, int k, u32x4 w) -> u32x4 {
    if (ti.wave && ti.slot == k) {  // uniform: one wave, one slot
      if (ti.mine) w = E::kill(w, tj);
    }
    if (k * NT + NT > pr.len) {
      // a branch, not selects on every slot: only a part's last slot can
      // reach past its end
      asm volatile("");
      constexpr unsigned n = E::kNegInfWord;
      const bool ok = tid < pr.len - k * NT;
      w = ok ? w : u32x4{n, n, n, n};
    }
    return w;
  };
  // Pass 1 state: the thread's maximum.  16-bit types keep packed integer
  // maxima (pk_max16) and fall back to packed minima when every element
  // is negative; fp32 keeps a float.
  struct MaxState {
    s16x2 hi;   // 16-bit: packed integer maximum
    s16x2 lo;   // 16-bit: packed integer minimum (second pass, all negative)
    float f;    // fp32
  };
  constexpr short kNegInfBits = (short)(E::kNegInfWord & 0xFFFFu);
  auto max_init = [&]() {
    return MaxState{s16x2{(short)-32768, (short)-32768}, s16x2{kNegInfBits, kNegInfBits}, kNegInf};
  };
  auto max_add = [&](MaxState& m, u32x4 w) {
    if constexpr (k16) {
      m.hi = __builtin_elementwise_max(m.hi, pk_max16(w));
    } else {
      const f32x4 x = as_f32(w);
      m.f = fmax3(fmax3(m.f, x.x, x.y), x.z, x.w);
    }
  };
  auto max_add_neg = [&](MaxState& m, u32x4 w) {
    if constexpr (k16) m.lo = __builtin_elementwise_min(m.lo, pk_min16(w));
  };
  // whether the second (all-negative) pass is needed, and the final value
  auto max_needs_neg = [&](const MaxState& m) -> bool {
    if constexpr (k16) return (m.hi.x > m.hi.y ? m.hi.x : m.hi.y) < 0;
    return false;
  };
  auto max_value = [&](const MaxState& m) -> float {
    if constexpr (k16) {
      const short h = m.hi.x > m.hi.y ? m.hi.x : m.hi.y;
      const short b = h >= 0 ? h : (m.lo.x < m.lo.y ? m.lo.x : m.lo.y);
      return widen_half<T>((unsigned)(unsigned short)b, 0);
    } else {
      return m.f;
    }
  };
  // c from a maximum over slots and, where the thread has one, its edge
  // element
  auto pair_c = [&](float m, int e, float x) -> float {
    if (e >= 0) m = fmax2(m, x);
    return fmax2(m * kLog2e, kLowest);
  };
  // The part that holds the target folds z_t into its pair's maximum (the
  // target stays out of the sum), so that the row's cg >= z_t log2 e.
  auto fold_target = [&](bool has_t, float zt_, float& cp_, float& sp_) {
    if (has_t) {
      const float cn = fmax2(cp_, zt_ * kLog2e);
      sp_ = sp_ * exp2_hw(cp_ - cn);
      cp_ = cn;
    }
  };
  // Pass 2 of one slot: its terms and their sum (the slot's words as from
  // slot_words).
  auto slot_terms = [&](u32x4 w, float c, float (&e)[VE]) -> float {
    float f[VE];
    E::unpack(w, f);
#pragma unroll
    for (int i = 0; i < VE; ++i) e[i] = exp2_hw(__builtin_fmaf(f[i], kLog2e, -c));
    return tree_sum(e);
  };
  auto edge_term = [&](int e, float x, float c) -> float {
    return (e >= 0 && e != t) ? exp2_hw(__builtin_fmaf(x, kLog2e, -c)) : 0.f;
  };

  // Phase B: this part's pair.
  constexpr bool kKeepTerms = sizeof(T) == 4 && !IP && (P <= 2 || (P == 4 && NL + NXW == 0));
  // Each phase tests the slots against its own opaque copy of the part's
  // length: conditions shared between phases would stay live in scalar
  // registers from pass 1 to the gradient, and the compiler spills them.
  auto opaque = [](int x) {
    asm volatile("" : "+s"(x));
    return x;
  };
  // 16-bit parts take c from their first slot alone and fold every slot
  // as soon as its data is in, so that the exponentials of the first slots
  // overlap the loads of the last.  A thread whose sum reaches 2^32 (an
  // element about 22 or more above its first slot's maximum, or a NaN)
  // forms it again from its true maximum.  Below that bound every element
  // lies at most 32 above its thread's c in log2 units, and so above the
  // row's cg: the row's Sx stays below C * 2^32 <= 2^60, and the loss's
  // Sx * 2^(-a_t) (taken while a_t > -60) below 2^120, with no overflow
  // anywhere after the sum.  fp32 parts, which keep their terms in the
  // register slots, take the maximum over all their slots first.
  constexpr bool kFirstSlotC = sizeof(T) == 2;
  constexpr float kFirstSlotSumMax = 0x1p32f;
  auto keep_terms = [&](int k, const float (&e)[VE]) {
    if constexpr (kKeepTerms) v[k] = as_u32(f32x4{e[0], e[1], e[2], e[3]});
    if constexpr (kLdsTerms > 0) {
      if (k < kLdsTerms) {
        kept[(2 * k) * NT + tid] = f32x4{e[0], e[1], e[2], e[3]};
        kept[(2 * k + 1) * NT + tid] = f32x4{e[4], e[5], e[6], e[7]};
      }
    }
  };
  // the thread's maximum over all its slots (slot_words already applied to
  // the register slots)
  auto full_max = [&](int len) -> float {
    MaxState ms = max_init();
#pragma unroll
    for (int k = 0; k < NR; ++k)
      if (k * NT < len) max_add(ms, v[k]);
#pragma unroll
    for (int p = 0; p < NLS; ++p)
      if ((NR + p) * NT < len) max_add(ms, slot_words(own, tin, NR + p, lds_slot(p)));
    if (max_needs_neg(ms)) {
#pragma unroll
      for (int k = 0; k < NR; ++k)
        if (k * NT < len) max_add_neg(ms, v[k]);
#pragma unroll
      for (int p = 0; p < NLS; ++p)
        if ((NR + p) * NT < len) max_add_neg(ms, slot_words(own, tin, NR + p, lds_slot(p)));
    }
    return max_value(ms);
  };
  // the sum over all slots (and the edge element) with a given c
  auto full_sum = [&](int len, float c_, float xs_) -> float {
    float s_ = 0.f;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      if (k * NT >= len) continue;
      float e[VE];
      s_ = s_ + slot_terms(v[k], c_, e);
      keep_terms(k, e);
    }
#pragma unroll
    for (int p = 0; p < NLS; ++p) {
      if ((NR + p) * NT >= len) continue;
      float e[VE];
      s_ = s_ + slot_terms(slot_words(own, tin, NR + p, lds_slot(p)), c_, e);
    }
    return s_ + edge_term(xe, xs_, c_);
  };
  float c, s;
  float xs;
  if constexpr (kFirstSlotC) {
    const int len = opaque(own.len);
    float c0 = kLowest;
    if (0 < len) {
      v[0] = slot_words(own, tin, 0, v[0]);
      MaxState m0 = max_init();
      max_add(m0, v[0]);
      if (max_needs_neg(m0)) max_add_neg(m0, v[0]);
      c0 = fmax2(max_value(m0) * kLog2e, kLowest);
    }
    s = 0.f;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      if (k * NT >= len) continue;
      if (k > 0) v[k] = slot_words(own, tin, k, v[k]);
      float e[VE];
      s = s + slot_terms(v[k], c0, e);
      keep_terms(k, e);
    }
    wait_vmcnt<0>();  // LDS slots (each thread reads its own wave's), edge and target loads
#pragma unroll
    for (int p = 0; p < NLS; ++p) {
      if ((NR + p) * NT >= len) continue;
      float e[VE];
      s = s + slot_terms(slot_words(own, tin, NR + p, lds_slot(p)), c0, e);
    }
    xs = xe >= 0 ? xs_raw : kNegInf;
    s = s + edge_term(xe, xs, c0);
    c = c0;
    if (!(s < kFirstSlotSumMax)) {  // an element far above c0 (or a NaN): the true maximum
      c = pair_c(full_max(len), xe, xs);
      s = full_sum(len, c, xs);
    }
  } else {
    const int len = opaque(own.len);
#pragma unroll
    for (int k = 0; k < NR; ++k)
      if (k * NT < len) v[k] = slot_words(own, tin, k, v[k]);
    wait_vmcnt<0>();  // LDS slots (each thread reads its own wave's), edge and target loads
    xs = xe >= 0 ? xs_raw : kNegInf;
    c = pair_c(full_max(len), xe, xs);
    s = full_sum(opaque(own.len), c, xs);
  }
  const float zt = t >= 0 ? zt_raw : 0.f;
  // The pairs of all parts, in LDS: this part's own, the others' as
  // received, or recomputed where a partner's did not arrive in time.
  float cg, sx;
  RowResult rr;
  if constexpr (P == 1) {
    wg_pair<NW>(c, s, red_c, red_s, lane, wv, cg, sx);
    fold_target(tin.part, zt, cg, sx);
    rr = row_finish<OP>(cg, sx, zt, valid, rt.ignored, invB, gmul);
    if (tid == 0) store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);
  } else {
    // Each wave's pair goes to LDS; wave 0 alone combines the 16, trades
    // the part's pair with its partners (thread 0) and, when every pair
    // has arrived, forms the row's results and leaves them in LDS (fin),
    // so the other waves run none of that arithmetic.
    wave_pair_to_lds(c, s, red_c, red_s, lane, wv);
    __syncthreads();
    // Eight parts keep the loops over partners rolled (less code, and no
    // partner's address or pair held beyond its iteration: the kernel is
    // capped at 64 VGPRs).
    constexpr int kUnrollPartners = P <= 4 ? P : 1;
    if (wv == 0) {
      float c_own, s_own;
      lds_pairs_combine<NW>(red_c, red_s, lane, c_own, s_own);
      fold_target(tin.part, zt, c_own, s_own);
      if (IP && P == 2 && tid == 0) {
        mail_c[part] = c_own;
        mail_s[part] = s_own;
        const int q = 1 - part;
        const uint64_t mw = in_place_word(c_own, s_own);
        uint64_t* const words = in_place + row * kInPlaceRowWords;
        uint64_t first = 0;
        int mode = 0;
        if (__hip_atomic_compare_exchange_strong(&words[0], &first, mw, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          // the first: the partner's pair comes to word 1
          uint64_t o = 0;
          for (int it = 0; it < spin; ++it) {
            o = __hip_atomic_load(&words[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (o != 0) break;
            __builtin_amdgcn_s_sleep(8);
          }
          if (o == 0 && __hip_atomic_compare_exchange_strong(&words[1], &o, kInPlaceDeferred,
                                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT)) {
            mode = 1;
          } else {
            in_place_pair(o, mail_c[q], mail_s[q]);
            __hip_atomic_store(&words[0], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&words[1], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          // the second: `first` holds the partner's pair
          in_place_pair(first, mail_c[q], mail_s[q]);
          uint64_t e = 0;
          if (!__hip_atomic_compare_exchange_strong(&words[1], &e, mw, __ATOMIC_RELAXED,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            mode = 2;  // the partner deferred: both halves are this part's to write
            __hip_atomic_store(&words[0], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&words[1], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        if (mode == 1 && fallbacks != nullptr) atomicAdd(fallbacks, 1u);
        ip_deferred = mode == 1 ? 1 : 0;
        ip_extra = mode == 2 ? 1u << q : 0u;
        mail_ok[0] = mail_ok[1] = 1;
        fin_ok = 1;
      } else if (IP && P > 2) {
        // Four or eight parts, on wave 0: lane q < P polls part q's pair
        // word and claims part q's flag, so that each pass over the words is
        // one access per lane; lane 0 publishes and counts.
        uint64_t* const words = in_place + row * kInPlaceRowWords;
        uint64_t* const flags = words + kInPlaceFlags;
        uint32_t* const arrived = reinterpret_cast<uint32_t*>(words + kInPlaceCounts);
        uint32_t* const departed = reinterpret_cast<uint32_t*>(words + kInPlaceCounts + 1);
        const bool watch = lane < P && lane != part;  // this lane waits for part `lane`'s pair
        uint32_t before = 0;
        if (lane == 0) {
          mail_c[part] = c_own;
          mail_s[part] = s_own;
          // publish, and wait until the word is written, then count the
          // arrival
          const uint64_t prev = __hip_atomic_exchange(&words[part], in_place_word(c_own, s_own),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          asm volatile("" ::"v"(prev) : "memory");
          before = __builtin_amdgcn_atomic_inc32(arrived, (uint32_t)(P - 1), __ATOMIC_RELAXED,
                                                 "agent");
        }
        before = __builtin_amdgcn_readfirstlane(before);
        bool have = !watch;
        // up to `polls` passes over the pair words (0: none)
        auto gather = [&](int polls) {
          for (int it = 0; it < polls; ++it) {
            if (!have) {
              const uint64_t x =
                  __hip_atomic_load(&words[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if (x != 0) {
                in_place_pair(x, mail_c[lane], mail_s[lane]);
                have = true;
              }
            }
            if (__builtin_amdgcn_ballot_w64(!have) == 0) break;
            __builtin_amdgcn_s_sleep(8);
          }
        };
        int deferred = 0;
        unsigned extra = 0;
        if (before == (uint32_t)(P - 1)) {
          // the closer: every other part has published
          gather(kInPlaceLongPolls);
          bool ext = false;
          if (watch) {
            uint64_t e = 0;
            ext = !__hip_atomic_compare_exchange_strong(&flags[lane], &e, kInPlaceChecked,
                                                        __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
          }
          extra = (unsigned)__builtin_amdgcn_ballot_w64(ext);  // e == kInPlaceDeferred
        } else {
          gather(spin);
          if (__builtin_amdgcn_ballot_w64(!have) != 0) {
            int d = 0;
            if (lane == 0) {
              uint64_t e = 0;
              d = __hip_atomic_compare_exchange_strong(&flags[part], &e, kInPlaceDeferred,
                                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT)
                      ? 1
                      : 0;
            }
            deferred = __builtin_amdgcn_readfirstlane(d);
            if (!deferred) gather(kInPlaceLongPolls);  // e == kInPlaceChecked: the closer has published
          }
        }
        if (!deferred && !have) {
          mail_c[lane] = __builtin_nanf("");  // a pair that never came: the row is NaN
          mail_s[lane] = __builtin_nanf("");
        }
        if (lane == 0) {
          // every access to the words above (the wave's polls and
          // compare-and-swaps) has completed before the departure counts
          wait_vmcnt<0>();
          if (__builtin_amdgcn_atomic_inc32(departed, (uint32_t)(P - 1), __ATOMIC_RELAXED, "agent") ==
              (uint32_t)(P - 1)) {
#pragma unroll 1
            for (int q = 0; q < P; ++q) {
              __hip_atomic_store(&words[q], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(&flags[q], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
          if (deferred && fallbacks != nullptr) atomicAdd(fallbacks, 1u);
          ip_deferred = deferred;
          ip_extra = extra;
#pragma unroll
          for (int q = 0; q < P; ++q) mail_ok[q] = 1;
          fin_ok = 1;
        }
      } else if (tid == 0) {
        mail_c[part] = c_own;
        mail_s[part] = s_own;
        const uint64_t tag = (uint64_t)kMailTag << 32;
        const uint64_t w0 = tag | __builtin_bit_cast(uint32_t, c_own);
        const uint64_t w1 = tag | __builtin_bit_cast(uint32_t, s_own);
        // The publishes are issued without waiting for their results, so
        // the next poll follows them at once.
        auto publish = [&] {
#pragma unroll kUnrollPartners
          for (int q = 0; q < P; ++q) {
            if (q == part) continue;
            uint64_t* m = mailbox(part_range(geo.nb, P, q)) + mail_index(part, q);
            uint64_t e0 = kEmptyWord, e1 = kEmptyWord;
            // a 64-bit compare-and-swap sends 16 bytes of data: the same
            // wait states as a wide store follow it
            __hip_atomic_compare_exchange_strong(&m[0], &e0, w0, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wide_store_guard();
            __hip_atomic_compare_exchange_strong(&m[1], &e1, w1, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wide_store_guard();
          }
        };
        publish();
        // a bit per part whose pair is here; received pairs go straight to LDS
        constexpr unsigned kAll = (1u << P) - 1u;
        unsigned got = 1u << part;
        bool behind = false;  // a pass has skipped its publish since the last one
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
          // Publish again on every fourth pass while pairs are missing; eight
          // parts also once more when the last pair arrives if a pass has
          // skipped since: every partner has then emptied its mailbox, which
          // may have wiped a pair sent before.
          const bool done = got == kAll;
          if (done ? (P == 8 && behind) : (it & 3) == 3) {
            publish();
            behind = false;
          } else {
            behind = !done;
          }
          if (!done) __builtin_amdgcn_s_sleep(8);
        }
#pragma unroll
        for (int q = 0; q < P; ++q) mail_ok[q] = (int)((got >> q) & 1u);
        fin_ok = got == kAll ? 1 : 0;
        if (got != kAll && fallbacks != nullptr)
          atomicAdd(fallbacks, (uint32_t)(P - __builtin_popcount(got)));
      }
      // wave 0 reads what its thread 0 wrote to LDS (in order, one wave)
      if (fin_ok) {
        combine_pairs<P>(mail_c, mail_s, cg, sx);
        rr = row_finish<OP>(cg, sx, zt, valid, rt.ignored, invB, gmul);
        // the loss goes with part 0's half (in place: with whoever writes it)
        const bool stores = IP ? (part == 0 ? !ip_deferred : (ip_extra & 1u) != 0) : part == 0;
        if (stores && tid == 0) store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);
        if (tid == 0) {
          fin[0] = cg;
          fin[1] = sx;
          fin[2] = rr.scale0;
          fin[3] = rr.scale;
          fin[4] = rr.gt;
        }
      }
    }
    __syncthreads();
    if constexpr (IP) {
      if (ip_deferred) return;  // uniform: a partner writes this part's gradient
    }
    if (fin_ok) {  // uniform (LDS, after the barrier): the common case
      cg = fin[0];
      sx = fin[1];
      rr.scale0 = fin[2];
      rr.scale = fin[3];
      rr.gt = fin[4];
    } else {
#pragma unroll kUnrollPartners
      for (int q = 0; q < P; ++q) {
        if (q == part || mail_ok[q]) continue;  // uniform (LDS, after the barrier)
        // Recompute part q's pair: the same slots, passes, edge and
        // workgroup reduction as part q runs itself, reading its logits
        // again for each pass.
        const PartRange pq = part_range(geo.nb, P, q);
        const rsrc_t rq = make_rsrc(rp + geo.h + pq.v0 * VE, (uint32_t)pq.len * 16u);
        const TargetIn tq = target_in(pq);
        auto load_q = [&](int k) {
          return slot_words(pq, tq, k, bload128<kPolicyStream>(rq, voff, (uint32_t)k * NT * 16u));
        };
        // (rolled loops: one slot's load in flight at a time, beside the
        // part's own slots held for its gradient)
        const int nq = (pq.len + NT - 1) / NT;  // slots holding part q's vectors
        const int xq = edge_elem(q);
        const float xqv = bload_elem<T>(rrow, (uint32_t)(xq >= 0 ? xq : C) * ES);
        const float xqs = xq >= 0 ? xqv : kNegInf;
        auto max_q = [&]() -> float {
          MaxState mq = max_init();
#pragma unroll 1
          for (int k = 0; k < nq; ++k) max_add(mq, load_q(k));
          if (max_needs_neg(mq)) {
#pragma unroll 1
            for (int k = 0; k < nq; ++k) max_add_neg(mq, load_q(k));
          }
          return max_value(mq);
        };
        auto sum_q = [&](float c_) -> float {
          float s_ = 0.f;
#pragma unroll 1
          for (int k = 0; k < nq; ++k) {
            float e[VE];
            s_ = s_ + slot_terms(load_q(k), c_, e);
          }
          return s_ + edge_term(xq, xqs, c_);
        };
        float cq, sq;
        if constexpr (kFirstSlotC) {
          float c0 = kLowest;
          if (0 < pq.len) {
            MaxState m0 = max_init();
            const u32x4 w0 = load_q(0);
            max_add(m0, w0);
            if (max_needs_neg(m0)) max_add_neg(m0, w0);
            c0 = fmax2(max_value(m0) * kLog2e, kLowest);
          }
          cq = c0;
          sq = sum_q(c0);
          if (!(sq < kFirstSlotSumMax)) {
            cq = pair_c(max_q(), xq, xqs);
            sq = sum_q(cq);
          }
        } else {
          cq = pair_c(max_q(), xq, xqs);
          sq = sum_q(cq);
        }
        float cr, sr;
        wg_pair<NW>(cq, sq, red_c, red_s, lane, wv, cr, sr);
        fold_target(tq.part, zt, cr, sr);
        if (tid == 0) {
          mail_c[q] = cr;
          mail_s[q] = sr;
        }
        __syncthreads();  // the pair is in LDS; red_c / red_s may be used again
      }
      combine_pairs<P>(mail_c, mail_s, cg, sx);
      rr = row_finish<OP>(cg, sx, zt, valid, rt.ignored, invB, gmul);
      if (part == 0 && tid == 0) store_row<OP>(loss_rows, row, rr, cg, sx, zt, t >= 0);
    }
  }

  // Phase C: the gradient of this part from registers and LDS.
#pragma unroll
  for (int k = 0; k < NR; ++k) asm volatile("" : "+v"(v[k]));
  if constexpr (kKeepTerms) {
    const float factor = exp2_hw(c - cg) * rr.scale;
    const int len = opaque(own.len);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      if (k * NT >= len) continue;
      const f32x4 e = as_f32(v[k]);
      const f32x4 g = {e.x * factor, e.y * factor, e.z * factor, e.w * factor};
      bstore128<kPolicyStream>(as_u32(g), rout, voff, (uint32_t)k * NT * 16u);
    }
    // LDS slots: the same terms formed again
#pragma unroll
    for (int p = 0; p < NLS; ++p) {
      if ((NR + p) * NT >= len) continue;
      float e[VE];
      slot_terms(slot_words(own, tin, NR + p, lds_slot(p)), c, e);
      const f32x4 g = {e[0] * factor, e[1] * factor, e[2] * factor, e[3] * factor};
      bstore128<kPolicyStream>(as_u32(g), rout, voff, (uint32_t)(NR + p) * NT * 16u);
    }
    if (xe >= 0)
      E::store1(gp + xe, xe == t ? rr.gt : exp2_hw(__builtin_fmaf(xs, kLog2e, -c)) * factor);
  } else {
    // 2^(z log2e - c') = 2^(z log2e - cg) / (S B); an ignored row has
    // 1/(S B) = 0, so c' = +inf and every element 0; an invalid one NaN
    const float cp = cg - log2_hw(rr.scale0);
    auto phase_c = [&](auto unit) {
      constexpr bool kUnit = decltype(unit)::value;
      auto grad_of = [&](float x) {
        const float g = exp2_hw(__builtin_fmaf(x, kLog2e, -cp));
        return kUnit ? g : g * gmul;
      };
      const int len = opaque(own.len);
      auto write_slot = [&](int k, u32x4 w) {
        if (k * NT >= len) return;
        float f[VE], g[VE];
        E::unpack(w, f);
#pragma unroll
        for (int i = 0; i < VE; ++i) g[i] = grad_of(f[i]);
        bstore128<kPolicyStream>(E::pack(g), rout, voff, (uint32_t)k * NT * 16u);
      };
      // slots whose terms 2^(z log2e - c) wait in LDS: times 2^(c - c')
      // (and gmul), the same value up to the rounding of one multiply
      if constexpr (kLdsTerms > 0) {
        // The kept terms are relative to the thread's c (its first slot's
        // maximum): where 2^(c - c') would lose precision below the normal
        // range, those slots are formed again from their logits.
        const float kfactor = kUnit ? exp2_hw(c - cp) : exp2_hw(c - cp) * gmul;
        const bool from_terms = c - cp >= -120.f;
#pragma unroll
        for (int k = 0; k < kLdsTerms; ++k) {
          if (k * NT >= len) continue;
          if (from_terms) {
            const f32x4 a = kept[(2 * k) * NT + tid], b = kept[(2 * k + 1) * NT + tid];
            const float g[VE] = {a.x * kfactor, a.y * kfactor, a.z * kfactor, a.w * kfactor,
                                 b.x * kfactor, b.y * kfactor, b.z * kfactor, b.w * kfactor};
            bstore128<kPolicyStream>(E::pack(g), rout, voff, (uint32_t)k * NT * 16u);
          } else {
            write_slot(k, v[k]);
          }
        }
      }
#pragma unroll
      for (int k = kLdsTerms; k < NR; ++k) write_slot(k, v[k]);
#pragma unroll
      for (int p = 0; p < NLS; ++p) write_slot(NR + p, lds_slot(p));
      if (xe >= 0) E::store1(gp + xe, xe == t ? rr.gt : grad_of(xs));
      if constexpr (IP) {
        // parts that deferred to this one: their logits are still there
#pragma unroll 1
        for (int q = 0; q < P; ++q) {
          if (!((ip_extra >> q) & 1u)) continue;  // uniform (LDS)
          const PartRange pq = part_range(geo.nb, P, q);
          const rsrc_t rq = make_rsrc(rp + geo.h + pq.v0 * VE, (uint32_t)pq.len * 16u);
          const rsrc_t rqo = make_rsrc(gp + geo.h + pq.v0 * VE, (uint32_t)pq.len * 16u);
          const int nq = (pq.len + NT - 1) / NT;
#pragma unroll 1
          for (int k = 0; k < nq; ++k) {
            float f[VE], g[VE];
            E::unpack(bload128<kPolicyStream>(rq, voff, (uint32_t)k * NT * 16u), f);
#pragma unroll
            for (int i = 0; i < VE; ++i) g[i] = grad_of(f[i]);
            bstore128<kPolicyStream>(E::pack(g), rqo, voff, (uint32_t)k * NT * 16u);
          }
          const int xq = edge_elem(q);
          if (xq >= 0) {
            const float x = bload_elem<T>(rrow, (uint32_t)xq * ES);
            E::store1(gp + xq, xq == t ? rr.gt : grad_of(x));
          }
          const TargetIn tq = target_in(pq);
          if (tq.k >= 0) E::store1(gp + geo.h + (int64_t)tvec * VE + tj, rr.gt);
        }
      }
    };
    if (gmul == 1.0f)
      phase_c(std::true_type{});
    else
      phase_c(std::false_type{});
  }
  // the target's gradient, over the value its vector store wrote there (the
  // same thread, the same address, later in program order)
  if (tin.k >= 0) E::store1(gp + geo.h + (int64_t)tvec * VE + tj, rr.gt);
}

}  // namespace ce
