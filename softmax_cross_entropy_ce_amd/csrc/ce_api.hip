// Host side of libce_mi355x.so: argument validation, path selection, launch
// geometry and the C ABI declared in include/ce.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>

#include "ce.h"
#include "ce_launch.h"
#include "ce_parts.h"
#include "ce_shard.h"
#include "softmax_bwd.h"
#include "softmax_bwd_parts.h"
#include "ce_wave_host.h"

namespace {

// Events for the next launch on this thread (ce_debug_time_next_launch).
thread_local hipEvent_t t_launch_start = nullptr;
thread_local hipEvent_t t_launch_stop = nullptr;

std::atomic<int> g_force_path{0};

constexpr int kPathShort = 1;
constexpr int kPathResident = 2;
constexpr int kPathLong = 3;
constexpr int kPathParts = 4;
constexpr int kPathWave = 5;

// Polls of a row part for its partner's pair before it recomputes the pair
// itself, and the optional device counter of such recomputations (test
// hooks; see ce_debug_part_polls / ce_debug_part_counter).
constexpr int kPartPollsDefault = 64;
std::atomic<int> g_part_polls{kPartPollsDefault};
std::atomic<uint32_t*> g_part_counter{nullptr};

// Per-row configurations of paths 2 and 3: NT threads, NV 16-byte vectors
// per thread, so NT*NV*16 bytes of the row stay in registers.  Ordered by
// capacity; the first that holds the row is taken.
struct RowCfg {
  int nt, nv;
};
constexpr RowCfg kRowCfgs[] = {{64, 1},   {64, 2},   {64, 4},    {256, 2},  {256, 4},
                               {1024, 2}, {1024, 4}, {1024, 8},  {1024, 16}};
// Rows read for a per-row value only (the loss alone, shard records) run on
// these: 256-thread workgroups hold up to 4096 vectors, so several rows
// are in flight on each compute unit (no gradient has to wait in
// registers for the row's reduction).
constexpr RowCfg kReadCfgs[] = {{64, 1},   {64, 2},   {64, 4},    {256, 2},  {256, 4},
                                {256, 8},  {256, 16}, {1024, 8},  {1024, 16}};
constexpr RowCfg kLongCfg = {1024, 16};     // automatic path 3 with a gradient
constexpr RowCfg kLongTestCfg = {256, 1};   // forced path 3: small on-chip part

constexpr int kShortMaxC = 256;
// Automatic selection (measured on rows filling 1 GiB): path 5 takes rows
// of up to 8 KB of 16-bit elements or 4 KB of float32; above that the
// one-part, 256-thread configuration of path 4 moved more bytes per second
// (the two crossed between 8 and 12 KB for bf16 rows, between 4 and 8 KB
// for fp32 rows).
// Rows path 5 has no configuration for stay on path 2 up to 256 vectors and
// go to path 4 above; longer rows go to path 4 while their aligned body
// fits its largest configuration, then to path 3.
constexpr int64_t kWaveAutoMaxBytes16 = 8192;
constexpr int64_t kWaveAutoMaxBytes32 = 4096;

int elem_size(int dtype) { return dtype == CE_F32 ? 4 : 2; }

// 16-byte vectors a row may touch: the aligned body plus a head and a tail.
int64_t row_vectors(int64_t C, int es) { return (C * es + 15) / 16 + 1; }

// Path 4 configurations by the largest body a row can have, floor(C /
// elements per vector) 16-byte vectors: one part of 256 threads and 8
// register slots (eight such workgroups fit a CU); one part of 1024
// threads and 4 register slots; one part of 8 register and 2 LDS slots;
// two parts of 8 register slots; two parts of 8 register and 4 LDS slots;
// four parts of 8 register slots; four parts of 8 register and 2 LDS
// slots; four parts of 8 register and 4 LDS slots (16-bit types; float32
// in place); eight parts of 8 register slots
// (a 1024-thread slot is 1024 vectors, and a part of a P-part row is 1/P of
// the body rounded up to 8 vectors).
constexpr int64_t kPartsOneQuarter = 8 * 256;
constexpr int64_t kPartsOneSmall = 4 * 1024;
constexpr int64_t kPartsOne = 10 * 1024;
constexpr int64_t kPartsTwoRegs = 2 * 8 * 1024;
constexpr int64_t kPartsTwo = 2 * 12 * 1024;
constexpr int64_t kPartsFourRegs = 4 * 8 * 1024;
constexpr int64_t kPartsFourLds2 = 4 * 10 * 1024;
constexpr int64_t kPartsFour = 4 * 12 * 1024;
constexpr int64_t kPartsEightRegs = 8 * 8 * 1024;
// The largest body path 4 takes: eight register-only parts.  (Four parts
// with 2 LDS slots serve rows up to kPartsFourLds2, whose parts they fill
// better than eight parts of 8 slots: fp32 rows of 151936 columns, 0.69 ->
// 0.72 of 8 TB/s out of place and 0.64 -> 0.71 in place; four parts with 4
// LDS slots serve 16-bit rows up to kPartsFour, and fp32 rows only in
// place: out of place, 2048 x 180000 fp32 measured 0.706 that way against
// 0.716 in eight parts, in place 0.70 against 0.66.  fp32 parts with LDS
// slots do not keep their terms, which would exceed 64 VGPRs.)
int64_t parts_max(int) { return kPartsEightRegs; }

int64_t body_vectors_max(int64_t C, int es) { return C / (16 / es); }

// Vector bytes of path 5 for contiguous rows from 16-byte aligned bases:
// the widest of 16, 8 and 4 that divides the row's bytes (0 if none).
int wave_vb_contiguous(int64_t C, int es) {
  for (int vb = 16; vb >= 4; vb /= 2)
    if ((C * es) % vb == 0) return vb;
  return 0;
}

// Longest row the staged kernel takes on path 2 (a chunk of at least
// eight rows).  Path 2 runs it for the rows path 5 has no vectors for
// (16-bit rows of odd length); where path 5 can take a row with 8- or
// 4-byte vectors it was as fast or faster above about 340 elements, and
// within a few percent below.
int64_t staged_max_c(int es) { return (int64_t)ce::kStagedChunkBytes / (8 * es); }

// Lanes per row of the staged softmax backward for rows of C elements: the
// smallest S of 8, 16, 32 with C <= 16 * S and a pass of 256 / S rows within
// half a staged chunk (0: none).
int staged_bwd_lanes(int64_t C, int es) {
  for (int S = 8; S <= 32; S *= 2)
    if (C <= 16 * S && (int64_t)(256 / S) * C * es <= ce::kStagedBwdChunkBytes) return S;
  return 0;
}

int auto_path(int64_t C, int es) {
  if (C <= kShortMaxC) return kPathShort;
  if (C * es <= (es == 4 ? kWaveAutoMaxBytes32 : kWaveAutoMaxBytes16)) {
    if (ce_wave::lane_bytes(C, es, wave_vb_contiguous(C, es)) != 0) return kPathWave;
    // rows path 5 has no vectors for (16-bit, odd length): path 2 up to 256
    // vectors, one row part beyond (measured on rows filling 1 GiB: 2001
    // bf16 elements 4.2 TB/s on path 2 against 3.8 as a part; 2047 elements
    // 2.9 against 3.8, 4095 elements 3.8 against 5.4)
    return row_vectors(C, es) <= 256 ? kPathResident : kPathParts;
  }
  if (body_vectors_max(C, es) <= parts_max(es)) return kPathParts;
  return kPathLong;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int launched() { return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_LAUNCH; }

// ------------------------------------------------------------------ path 1
// Row groups per workgroup: lanes holding 16 bytes of a row take four rows
// each (their loads all issued first), 32 bytes two, more one.
template <typename T, int EPL>
constexpr int short_groups() {
  return EPL * (int)sizeof(T) <= 16 ? 4 : EPL * (int)sizeof(T) <= 32 ? 2 : 1;
}

template <typename T, int S, int EPL, int VW, int OP, bool GRAD>
int launch_short_cfg(const T* z, const int32_t* t, int64_t B, int C, ce::RowArgs rs, T* g, float* l,
                     hipStream_t st) {
  constexpr int R = short_groups<T, EPL>();
  constexpr int rpb = ce::kShortThreads / S * R;
  const int64_t blocks = (B + rpb - 1) / rpb;
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  ce_host::launch((ce::ce_short_kernel<T, S, EPL, VW, GRAD, OP, R>), dim3((unsigned)blocks),
                     dim3(ce::kShortThreads), 0, st, z, t, B, C, rs, g, l);
  return launched();
}

template <typename T, int S, int EPL, int OP, bool GRAD>
int launch_short_vw(int vw, const T* z, const int32_t* t, int64_t B, int C, ce::RowArgs rs, T* g,
                    float* l, hipStream_t st) {
  switch (vw) {
    case 1: return launch_short_cfg<T, S, EPL, 1, OP, GRAD>(z, t, B, C, rs, g, l, st);
    case 2: return launch_short_cfg<T, S, EPL, 2, OP, GRAD>(z, t, B, C, rs, g, l, st);
    case 4: return launch_short_cfg<T, S, EPL, 4, OP, GRAD>(z, t, B, C, rs, g, l, st);
    case 8:
      if constexpr (sizeof(T) == 2 && EPL >= 8)
        return launch_short_cfg<T, S, EPL, 8, OP, GRAD>(z, t, B, C, rs, g, l, st);
      return CE_ERR_PATH;
    default: return CE_ERR_PATH;
  }
}

// Vector width (elements) of the short path: the widest load of at most 16
// bytes that every row start of both arrays is aligned to (lens: the row
// length and both row strides, each a multiple of the width).
int short_vw(int64_t lens, int es, uintptr_t zaddr, uintptr_t gaddr, int epl) {
  for (int vw = 16 / es; vw > 1; vw /= 2) {
    const uintptr_t a = (uintptr_t)vw * es;
    if (vw <= epl && lens % vw == 0 && zaddr % a == 0 && gaddr % a == 0) return vw;
  }
  return 1;
}

// The short path addresses a workgroup's up to 1024 rows (256 segments of
// one lane, four groups) through one buffer resource per array: their span
// must stay below 2^31 bytes.
bool short_span_ok(int64_t C, int64_t ld, int es) {
  return C <= kShortMaxC && (1023 * ld + C) * es < ((int64_t)1 << 31);
}

int resident_blocks(const void* kernel, int nt, std::atomic<int>& per_cu_cache);

// Rows of at most 64 bytes, contiguous, in 16-byte aligned arrays: the
// LDS-staged kernel, one chunk of 64 * R rows per wave (R rows per lane,
// below), four waves per workgroup.  Rows of more than 32 bytes take one
// per lane.
constexpr int kTinyRowsPerThread = 1;

template <typename T, int CMAX, int R, int OP, bool GRAD, bool PAD>
int launch_tiny_w(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                  float* l, hipStream_t st) {
  auto kern = ce::ce_tiny_kernel<T, CMAX, R, GRAD, OP, PAD>;
  const int64_t rows = (int64_t)ce::kTinyThreads * R;   // rows of one workgroup's four chunks
  const int64_t grid = (B + rows - 1) / rows;            // B < 2^31: at most 2^23 workgroups
  ce_host::launch(kern, dim3((unsigned)grid), dim3(ce::kTinyThreads), 0, st, z, t, B, (int)C, rs,
                  g, l);
  return launched();
}

// Rows of a multiple of 16 bytes (4, 8, 12 or 16 words) take the padded
// LDS layout: at their own stride the threads of a wave, each reading its
// row, would meet 4- to 16-way bank conflicts.  Other rows keep the packed
// layout, whose conflicts are at most 2-way (an odd number of words, or
// 2, 6, 10 or 14) and where the padded layout's address arithmetic and
// registers cost more than it saves (measured: 2,097,152 x 10 fp32 rows
// 37.0 us packed against 39.3 us padded).
template <typename T, int CMAX, int R, int OP, bool GRAD>
int launch_tiny_p(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                  float* l, hipStream_t st) {
  if ((C * (int64_t)sizeof(T)) % 16 == 0)
    return launch_tiny_w<T, CMAX, R, OP, GRAD, true>(z, t, B, C, rs, g, l, st);
  return launch_tiny_w<T, CMAX, R, OP, GRAD, false>(z, t, B, C, rs, g, l, st);
}

// Rows per lane: 16-bit rows of at most 8 elements take four per lane, other
// rows of at most 32 bytes two, longer rows one, so that a wave's chunk
// (and the loads in flight) is not a few hundred bytes.  Measured on rows
// filling 256 MB, GB/s of logits and gradient for one, two and four rows
// per lane: fp32 C = 2: 2033, 2520, 2329; fp32 C = 6: 4831, 5450, 4981;
// fp32 C = 8: 5767, 5989, 5355; bf16 C = 4: 2052, 2467, 2744; bf16 C = 8:
// 3612, 4172, 4367 (a copy of the same bytes: 6080-6180).
template <typename T, int CMAX, int OP, bool GRAD>
int launch_tiny_c(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                  float* l, hipStream_t st) {
  if constexpr (sizeof(T) == 2 && CMAX == 8) {
    return launch_tiny_p<T, CMAX, 4, OP, GRAD>(z, t, B, C, rs, g, l, st);
  } else if constexpr (CMAX * sizeof(T) <= 32) {
    return launch_tiny_p<T, CMAX, 2, OP, GRAD>(z, t, B, C, rs, g, l, st);
  } else {
    return launch_tiny_p<T, CMAX, kTinyRowsPerThread, OP, GRAD>(z, t, B, C, rs, g, l, st);
  }
}

template <typename T, int OP, bool GRAD>
int launch_tiny(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g, float* l,
                hipStream_t st) {
  if (C <= 8) return launch_tiny_c<T, 8, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 12) return launch_tiny_c<T, 12, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 16) return launch_tiny_c<T, 16, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if constexpr (sizeof(T) == 2) return launch_tiny_c<T, 32, OP, GRAD>(z, t, B, C, rs, g, l, st);
  return CE_ERR_PATH;
}

template <typename T>
bool tiny_rows(const T* z, int64_t C, const ce::RowArgs& rs, const T* g, bool grad) {
  return C * (int64_t)sizeof(T) <= ce::kTinyRowBytes && rs.ldz == C && (uintptr_t)z % 16 == 0 &&
         (!grad || (rs.ldg == C && (uintptr_t)g % 16 == 0));
}

// Contiguous rows in 16-byte aligned arrays whose byte length 16 does not
// divide (the short kernel would read them with narrower loads): the
// LDS-staged kernel, persistent over chunks of rows, with the short
// kernel's segment layout.  It takes them from 33 bytes for 16-bit types
// (two lanes per row beat the tiny kernel's one thread per row from 17
// elements on) and from 65 bytes for fp32 (the tiny kernel up to 16
// elements).
template <typename T>
constexpr int64_t kStagedMinBytes = sizeof(T) == 2 ? 32 : ce::kTinyRowBytes;
template <typename T>
bool staged_rows(const T* z, int64_t C, const ce::RowArgs& rs, const T* g, bool grad) {
  return C * (int64_t)sizeof(T) > kStagedMinBytes<T> && (C * (int64_t)sizeof(T)) % 16 != 0 &&
         rs.ldz == C && (uintptr_t)z % 16 == 0 &&
         (!grad || (rs.ldg == C && (uintptr_t)g % 16 == 0));
}

template <typename T, int S, int EPL, int OP, bool GRAD>
int launch_staged_cfg(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                      float* l, hipStream_t st) {
  auto kern = ce::ce_staged_kernel<T, S, EPL, GRAD, OP>;
  static std::atomic<int> occupancy{0};
  const int res = resident_blocks(reinterpret_cast<const void*>(kern), ce::kStagedThreads, occupancy);
  if (res < 1) return CE_ERR_LAUNCH;
  const int64_t rows = ce::staged_rows_per_chunk((int)C, (int)sizeof(T), ce::kStagedThreads / S);
  if (rows < 1 || C > S * EPL) return CE_ERR_PATH;  // a chunk pass and the slots hold a row
  const int64_t chunks = (B + rows - 1) / rows;
  const int64_t grid = chunks < res ? chunks : res;
  ce_host::launch(kern, dim3((unsigned)grid), dim3(ce::kStagedThreads), 0, st, z, t, B, (int)C,
                     rs, g, l);
  return launched();
}

// Two lanes per row up to 32 fp32 or 64 16-bit elements (rows of at most
// 128 bytes, so that a pass of 128 rows fits a chunk), four up to 64 (96
// for 16-bit types), eight up to 128, sixteen up to 256: fewer lanes per
// row let more rows share each reduction step.  Slots per lane in steps
// that leave at most about a fifth of them past the row's end (rows of
// more than 64 bytes: C > 16 for fp32, C > 32 for 16-bit types).  With
// eight lanes, fp32 rows of 17-49 elements ran at 50-84 % of a copy's rate
// and bf16 rows of 33-91 at 41-72 %; with two or four, 86-94 % and 70-83 %.
// From 97 bf16 elements on, eight lanes were faster.
template <typename T, int OP, bool GRAD>
int launch_staged(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                  float* l, hipStream_t st) {
  if (C <= 32) return launch_staged_cfg<T, 2, 16, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if constexpr (sizeof(T) == 2) {
    if (C <= 40) return launch_staged_cfg<T, 2, 20, OP, GRAD>(z, t, B, C, rs, g, l, st);
    if (C <= 48) return launch_staged_cfg<T, 2, 24, OP, GRAD>(z, t, B, C, rs, g, l, st);
    if (C <= 56) return launch_staged_cfg<T, 2, 28, OP, GRAD>(z, t, B, C, rs, g, l, st);
    if (C <= 64) return launch_staged_cfg<T, 2, 32, OP, GRAD>(z, t, B, C, rs, g, l, st);
  }
  if (C <= 40) return launch_staged_cfg<T, 4, 10, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 48) return launch_staged_cfg<T, 4, 12, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 64) return launch_staged_cfg<T, 4, 16, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if constexpr (sizeof(T) == 2) {
    if (C <= 80) return launch_staged_cfg<T, 4, 20, OP, GRAD>(z, t, B, C, rs, g, l, st);
    if (C <= 96) return launch_staged_cfg<T, 4, 24, OP, GRAD>(z, t, B, C, rs, g, l, st);
  }
  if (C <= 80) return launch_staged_cfg<T, 8, 10, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 96) return launch_staged_cfg<T, 8, 12, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 112) return launch_staged_cfg<T, 8, 14, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 128) return launch_staged_cfg<T, 8, 16, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 160) return launch_staged_cfg<T, 16, 10, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 192) return launch_staged_cfg<T, 16, 12, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 224) return launch_staged_cfg<T, 16, 14, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 256) return launch_staged_cfg<T, 16, 16, OP, GRAD>(z, t, B, C, rs, g, l, st);
  return CE_ERR_PATH;
}

// 16-bit rows of 257 to 1024 elements on path 2 (a chunk holds at least
// eight rows): 32 lanes per row, slots in steps that waste at most a fifth
// of them.

template <typename T, int OP, bool GRAD>
int launch_staged_long(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                       float* l, hipStream_t st) {
  static_assert(sizeof(T) == 2, "fp32 rows of this length have path 5");
  if (C <= 320) return launch_staged_cfg<T, 32, 10, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 384) return launch_staged_cfg<T, 32, 12, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 512) return launch_staged_cfg<T, 32, 16, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 640) return launch_staged_cfg<T, 32, 20, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 768) return launch_staged_cfg<T, 32, 24, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (C <= 1024) return launch_staged_cfg<T, 32, 32, OP, GRAD>(z, t, B, C, rs, g, l, st);
  return CE_ERR_PATH;
}

// Short-row layout: about 16 bytes per lane.  S lanes per row is the power
// of two that covers the row with EPL elements per lane (EPL = 16 bytes of
// elements, more only at S = 16).  Lanes of a row read adjacent vectors,
// so a load instruction covers 64/S consecutive rows.
template <typename T, int OP, bool GRAD>
int launch_short(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g, float* l,
                 hipStream_t st) {
  if (staged_rows(z, C, rs, g, GRAD)) return launch_staged<T, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (tiny_rows(z, C, rs, g, GRAD)) return launch_tiny<T, OP, GRAD>(z, t, B, C, rs, g, l, st);
  if (!short_span_ok(C, rs.ldz, sizeof(T)) || (GRAD && !short_span_ok(C, rs.ldg, sizeof(T))))
    return CE_ERR_PATH;
  constexpr int es = sizeof(T);
  constexpr int E16 = 16 / es;  // elements in 16 bytes
  const int c = (int)C;
  const int64_t lens = C | rs.ldz | (GRAD ? rs.ldg : 0);
  auto vw = [&](int epl) { return short_vw(lens, es, (uintptr_t)z, (uintptr_t)g, epl); };
  if (C <= E16) return launch_short_vw<T, 1, E16, OP, GRAD>(vw(E16), z, t, B, c, rs, g, l, st);
  if (C <= 2 * E16) return launch_short_vw<T, 2, E16, OP, GRAD>(vw(E16), z, t, B, c, rs, g, l, st);
  if (C <= 4 * E16) return launch_short_vw<T, 4, E16, OP, GRAD>(vw(E16), z, t, B, c, rs, g, l, st);
  if (C <= 8 * E16) return launch_short_vw<T, 8, E16, OP, GRAD>(vw(E16), z, t, B, c, rs, g, l, st);
  if (C <= 16 * E16) return launch_short_vw<T, 16, E16, OP, GRAD>(vw(E16), z, t, B, c, rs, g, l, st);
  if constexpr (E16 < 16) {
    if (C <= 32 * E16)
      return launch_short_vw<T, 16, 2 * E16, OP, GRAD>(vw(2 * E16), z, t, B, c, rs, g, l, st);
  }
  if constexpr (E16 < 8) {
    if (C <= 64 * E16)
      return launch_short_vw<T, 16, 4 * E16, OP, GRAD>(vw(4 * E16), z, t, B, c, rs, g, l, st);
  }
  return CE_ERR_PATH;
}

// -------------------------------------------------------------- paths 2, 3
// Workgroups of a kernel that the current device holds at once: compute
// units times the occupancy of that kernel.  The row kernels are persistent,
// so their grid is this number (or B when that is smaller).
// The compute-unit count is cached per device (a partitioned GPU exposes
// devices of fewer units) and the occupancy per kernel by the caller, so a
// launch queries the runtime only the first time.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && (cus = g_device_cus[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  if (cached) g_device_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int resident_blocks(const void* kernel, int nt, std::atomic<int>& per_cu_cache) {
  const int cus = device_cus();
  if (cus < 1) return -1;
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu < 1) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nt, 0) != hipSuccess)
      return -1;
    if (per_cu < 1) per_cu = 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  return cus * per_cu;
}

// 16-bit rows read for their per-row value with 8 register slots (the
// streaming read configurations): at most seven waves per SIMD.  At 63
// VGPRs the kernel fits eight, and the extra workgroups slowed the streams
// (measured: the loss alone on 8192 x 128256 bf16, 512 x 8, took 378 us
// with four workgroups per CU against 333 us with three).
constexpr int kReadWavesPerSimd = 7;

template <typename T, int NT, int NV, int OP, bool GRAD>
int launch_row_cfg(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                   float* l, hipStream_t st) {
  auto kern = ce::ce_row_kernel<T, NT, NV, GRAD, OP>;
  static std::atomic<int> occupancy{0};
  int res = resident_blocks(reinterpret_cast<const void*>(kern), NT, occupancy);
  if (res < 1) return CE_ERR_LAUNCH;
  if constexpr (!GRAD && sizeof(T) == 2 && NV == 8) {
    constexpr int kPerCu = kReadWavesPerSimd * 4 / (NT / 64) > 0 ? kReadWavesPerSimd * 4 / (NT / 64) : 1;
    const int cap = device_cus() * kPerCu;
    if (cap > 0 && res > cap) res = cap;
  }
  const int64_t grid = B < res ? B : res;
  ce_host::launch(kern, dim3((unsigned)grid), dim3(NT), 0, st, z, t, B, (int)C, rs, g, l);
  return launched();
}

// Rows that need the largest register configuration run the variant with
// the next row's prefix prefetched into LDS.
constexpr int kLdsPrefetchSlots = 9;  // 9 x 16 KB of the 160 KB of LDS

template <typename T, int OP>
int launch_row_lds(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                   float* l, hipStream_t st) {
  auto kern = ce::ce_row_lds_kernel<T, 16, kLdsPrefetchSlots, OP>;
  static std::atomic<int> occupancy{0};
  const int res = resident_blocks(reinterpret_cast<const void*>(kern), 1024, occupancy);
  if (res < 1) return CE_ERR_LAUNCH;
  const int64_t grid = B < res ? B : res;
  ce_host::launch(kern, dim3((unsigned)grid), dim3(1024), 0, st, z, t, B, (int)C, rs, g, l);
  return launched();
}

template <typename T, int OP, bool GRAD>
int launch_row(RowCfg cfg, const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
               float* l, hipStream_t st) {
#define CE_ROW_CASE(NT_, NV_)                                                           \
  if (cfg.nt == NT_ && cfg.nv == NV_)                                                   \
    return launch_row_cfg<T, NT_, NV_, OP, GRAD>(z, t, B, C, rs, g, l, st);
  CE_ROW_CASE(64, 1)
  CE_ROW_CASE(64, 2)
  CE_ROW_CASE(64, 4)
  CE_ROW_CASE(256, 1)
  CE_ROW_CASE(256, 2)
  CE_ROW_CASE(256, 4)
  if constexpr (!GRAD) {
    CE_ROW_CASE(128, 16)
    CE_ROW_CASE(256, 8)
    CE_ROW_CASE(256, 16)
    CE_ROW_CASE(512, 8)
  }
  CE_ROW_CASE(1024, 2)
  CE_ROW_CASE(1024, 4)
  CE_ROW_CASE(1024, 8)
  CE_ROW_CASE(1024, 16)
#undef CE_ROW_CASE
  return CE_ERR_PATH;
}

// 16-byte vectors of a row's body: exactly floor(C * es / 16) when every
// row of every array starts on a 16-byte boundary, else at most
// row_vectors.
int64_t row_need(int64_t C, int es, bool aligned) {
  return aligned ? C * es / 16 : row_vectors(C, es);
}

RowCfg resident_cfg(int64_t C, int es, bool* ok, bool grad = true, bool aligned = false) {
  const int64_t need = row_need(C, es, aligned);
  for (const RowCfg& r : (grad ? kRowCfgs : kReadCfgs))
    if ((int64_t)r.nt * r.nv >= need) {
      *ok = true;
      return r;
    }
  *ok = false;
  return kLongCfg;
}

// Automatic configuration of a row read for its per-row value only, by the
// 16-byte vectors it needs.  Up to 4096 vectors (16-bit types, but see the
// rows of 65 to 1024 vectors below) or 1024 (float32) the first of
// kReadCfgs that holds the row; longer rows keep a
// part of the row on chip and stream the rest, in the configuration that
// moved the most bytes per second on rows filling 1 GiB: 16-bit rows with
// 256 threads x 8 slots up to 12288 vectors and 512 x 8 beyond (the
// 1024-thread configurations that hold such rows whole fit one workgroup
// per compute unit and left it idle while a row is reduced); float32 rows
// with 128 x 16 up to 6144 vectors and 1024 x 4 beyond.
RowCfg read_cfg(int64_t need, int es) {
  if (es == 2) {
    if (need > 12288) return {512, 8};
    if (need > 4096) return {256, 8};
    // 16-bit rows of up to 16 KB reach here when path 5 has no vectors for
    // them (odd lengths, strides or bases): one wave per row, streaming past
    // 4 vectors per lane, moved 3.7-5.6 TB/s on odd rows of 1025-4095 bf16
    // elements against 1.1-3.6 for the 256-thread configurations that hold
    // them
    if (need > 64 && need <= 1024) return {64, 4};
  } else {
    if (need > 6144) return {1024, 4};
    if (need > 1024) return {128, 16};
  }
  for (const RowCfg& r : kReadCfgs)
    if ((int64_t)r.nt * r.nv >= need) return r;
  return kLongCfg;
}

// ---------------------------------------------------------------- path 4
template <typename T, int P, int NT, int NR, int NL, int NXW, int OP, bool IP = false>
int launch_parts_cfg(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g,
                     float* l, hipStream_t st, uint64_t* in_place = nullptr) {
  const int64_t blocks = P * ((B + 7) / 8 * 8);
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  ce_host::launch((ce::ce_part_kernel<T, P, NT, NR, NL, NXW, OP, IP>), dim3((unsigned)blocks),
                  dim3(NT), 0, st, z, t, B, (int)C, rs, g, l,
                  g_part_polls.load(std::memory_order_relaxed),
                  g_part_counter.load(std::memory_order_relaxed), in_place);
  return launched();
}

template <typename T, int OP>
int launch_parts(const T* z, const int32_t* t, int64_t B, int64_t C, ce::RowArgs rs, T* g, float* l,
                 hipStream_t st, uint64_t* in_place = nullptr) {
  const int64_t nb = body_vectors_max(C, sizeof(T));
  if (in_place != nullptr) {  // rows of several parts in place, the same parts as out of place
    if constexpr (OP == ce::kOpCE) {
      if (nb <= kPartsOne) return CE_ERR_PATH;
      if (nb <= kPartsTwoRegs)
        return launch_parts_cfg<T, 2, 1024, 8, 0, 0, OP, true>(z, t, B, C, rs, g, l, st, in_place);
      if (nb <= kPartsTwo)
        return launch_parts_cfg<T, 2, 1024, 8, 4, 0, OP, true>(z, t, B, C, rs, g, l, st, in_place);
      if (nb <= kPartsFourRegs)
        return launch_parts_cfg<T, 4, 1024, 8, 0, 0, OP, true>(z, t, B, C, rs, g, l, st, in_place);
      if (nb <= kPartsFourLds2)
        return launch_parts_cfg<T, 4, 1024, 8, 2, 0, OP, true>(z, t, B, C, rs, g, l, st, in_place);
      if (nb <= kPartsFour)
        return launch_parts_cfg<T, 4, 1024, 8, 4, 0, OP, true>(z, t, B, C, rs, g, l, st, in_place);
      if (nb <= kPartsEightRegs)
        return launch_parts_cfg<T, 8, 1024, 8, 0, 0, OP, true>(z, t, B, C, rs, g, l, st, in_place);
    }
    return CE_ERR_PATH;
  }
  if (nb <= kPartsOneQuarter) return launch_parts_cfg<T, 1, 256, 8, 0, 0, OP>(z, t, B, C, rs, g, l, st);
  if (nb <= kPartsOneSmall) return launch_parts_cfg<T, 1, 1024, 4, 0, 0, OP>(z, t, B, C, rs, g, l, st);
  if (nb <= kPartsOne) return launch_parts_cfg<T, 1, 1024, 8, 2, 0, OP>(z, t, B, C, rs, g, l, st);
  if (nb <= kPartsTwoRegs) return launch_parts_cfg<T, 2, 1024, 8, 0, 0, OP>(z, t, B, C, rs, g, l, st);
  if (nb <= kPartsTwo) return launch_parts_cfg<T, 2, 1024, 8, 4, 0, OP>(z, t, B, C, rs, g, l, st);
  if (nb <= kPartsFourRegs) return launch_parts_cfg<T, 4, 1024, 8, 0, 0, OP>(z, t, B, C, rs, g, l, st);
  if (nb <= kPartsFourLds2) return launch_parts_cfg<T, 4, 1024, 8, 2, 0, OP>(z, t, B, C, rs, g, l, st);
  if constexpr (sizeof(T) == 2) {
    if (nb <= kPartsFour) return launch_parts_cfg<T, 4, 1024, 8, 4, 0, OP>(z, t, B, C, rs, g, l, st);
  }
  if (nb <= kPartsEightRegs) return launch_parts_cfg<T, 8, 1024, 8, 0, 0, OP>(z, t, B, C, rs, g, l, st);
  return CE_ERR_PATH;
}

// GRAD false: the per-row output only, on the short, resident or long path
// (nothing has to stay on chip for a gradient, so no row parts).
template <typename T, int OP, bool GRAD>
int fwd_typed(int path, const T* z, const int32_t* t, int64_t B, int64_t C, T* g, float* l,
              ce::RowArgs rs, hipStream_t st, uint64_t* in_place = nullptr) {
  constexpr int es = sizeof(T);
  const bool aligned = (uintptr_t)z % 16 == 0 && (rs.ldz * es) % 16 == 0 &&
                       (!GRAD || ((uintptr_t)g % 16 == 0 && (rs.ldg * es) % 16 == 0));
  const bool forced = g_force_path.load(std::memory_order_relaxed) != 0;
  switch (path) {
    case kPathShort:
      return launch_short<T, OP, GRAD>(z, t, B, C, rs, g, l, st);
    case kPathResident: {
      bool ok = false;
      const RowCfg cfg = resident_cfg(C, es, &ok, GRAD, aligned);
      if (!ok) return CE_ERR_PATH;
      if constexpr (es == 2) {
        if (!forced && C > kShortMaxC && C <= staged_max_c(es) && staged_rows(z, C, rs, g, GRAD))
          return launch_staged_long<T, OP, GRAD>(z, t, B, C, rs, g, l, st);
      }
      if constexpr (GRAD) {
        if (cfg.nt == 1024 && cfg.nv == 16) return launch_row_lds<T, OP>(z, t, B, C, rs, g, l, st);
      } else {
        if (!forced) return launch_row<T, OP, GRAD>(read_cfg(row_need(C, es, aligned), es), z, t, B,
                                                    C, rs, g, l, st);
      }
      return launch_row<T, OP, GRAD>(cfg, z, t, B, C, rs, g, l, st);
    }
    case kPathLong: {
      if (forced) return launch_row<T, OP, GRAD>(kLongTestCfg, z, t, B, C, rs, g, l, st);
      return launch_row<T, OP, GRAD>(GRAD ? kLongCfg : read_cfg(row_need(C, es, aligned), es), z, t,
                                     B, C, rs, g, l, st);
    }
    case kPathParts:
      if constexpr (GRAD) return launch_parts<T, OP>(z, t, B, C, rs, g, l, st, in_place);
      return CE_ERR_PATH;
    default:
      return CE_ERR_PATH;
  }
}

// Rows that path 4 cuts into several parts: their parts may read each
// other's logits (the recompute) and keep mailboxes in grad, so in place
// they run on the in-place variant of the part kernel, and only when
// ce_fwd_grad_ex is given the rows' words (ce_fwd_inplace_workspace_bytes).
bool multi_part_row(int64_t C, int es) { return body_vectors_max(C, es) > kPartsOne; }

// The in-place rows' words in a ce_fwd_grad_ex workspace: a block of
// ce::kInPlaceRowWords 64-bit words a row from byte kInPlaceWordsOffset (the
// ignore_index count sits at byte 0), or null when the workspace is
// missing, too small or not 8-byte aligned.
constexpr size_t kInPlaceWordsOffset = 256;
constexpr size_t kInPlaceRowBytes = 8 * (size_t)ce::kInPlaceRowWords;
uint64_t* in_place_words(void* ws, size_t ws_bytes, int64_t B) {
  if (ws == nullptr || (uintptr_t)ws % 8 != 0) return nullptr;
  if (ws_bytes < kInPlaceWordsOffset + (size_t)B * kInPlaceRowBytes) return nullptr;
  return reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + kInPlaceWordsOffset);
}

// Rows that do not run as row parts (the loss alone, rows of several parts
// in place): path 5 where it has a configuration for contiguous rows (it falls
// back to path 2 at launch when the arrays do not allow it), else path 2 or
// 3 by length.
int path_without_parts(int64_t C, int es, bool grad) {
  if (C <= kShortMaxC) return kPathShort;
  if (ce_wave::lane_bytes(C, es, wave_vb_contiguous(C, es)) != 0) return kPathWave;
  const int64_t need = row_vectors(C, es);
  const RowCfg cap = grad ? kLongCfg : read_cfg(need, es);
  return need <= (int64_t)cap.nt * cap.nv ? kPathResident : kPathLong;
}

// Kept-row count of ignore_index: one workgroup for up to one round of
// targets (a single launch, all loads in flight at once), else one
// workgroup per round up to 256, after the zeroing launch.
constexpr int64_t kCountOneRows = ce::kCountRound;
constexpr int64_t kCountMaxBlocks = 256;

bool overlaps(uintptr_t a, uintptr_t an, uintptr_t b, uintptr_t bn) {
  return a < b + bn && b < a + an;
}

// ------------------------------------------------------------ reduction
// Up to kReduceOneLaunch rows one workgroup sums them in a single launch.
// Above, the first level has up to kReduceMaxBlocks workgroups with chunks
// of whole rounds of ce::kReduceRound rows (2048: eight per thread, all
// loaded at once), so that the whole GPU reads the rows in as few rounds as
// possible, then one workgroup sums the partials.
constexpr int64_t kReduceOneLaunch = 16384;
static_assert(kReduceOneLaunch == ce::kReduceOneMax, "one launch sums what one workgroup holds");
constexpr int64_t kReduceMaxBlocks = 1024;
constexpr int kMaxDevicesReduce = 64;
// a first-level chunk's bytes must fit the 32-bit range of a buffer resource
constexpr int64_t kReduceMaxChunk = (int64_t)1 << 29;
constexpr int64_t kReduceMaxRows = kReduceMaxChunk * kReduceMaxBlocks;

int64_t reduce_chunk(int64_t B) {
  if (B <= kReduceOneLaunch) return kReduceOneLaunch;
  const int64_t step = ce::kReduceRound;
  const int64_t chunk = (B + kReduceMaxBlocks - 1) / kReduceMaxBlocks;
  return (chunk + step - 1) / step * step;
}

int64_t reduce_blocks(int64_t B) { return (B + reduce_chunk(B) - 1) / reduce_chunk(B); }

// Launch the reduction of B per-row values into *out: one workgroup up to
// kReduceOneLaunch rows, else a first level of reduce_blocks(B) workgroups
// writing their partial sums into part, then one workgroup over those.
int launch_reduce(const float* rows, int64_t B, float* out, float* part, hipStream_t st);

// Device scratch of ce_reduce_loss_noalloc: the first level's partial sums,
// kReduceMaxBlocks floats (4 KB), one copy per GPU for the life of the
// process.  Host code never uses the array's name as a device address: the
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and is cached here per device.
__device__ __align__(256) float reduce_scratch[kReduceMaxBlocks];
std::atomic<float*> g_reduce_scratch[kMaxDevicesReduce];
std::mutex g_reduce_scratch_mu;

// The current device's copy of reduce_scratch; CE_ERR_LAUNCH when the
// runtime cannot give its address.
int reduce_scratch_ptr(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevicesReduce) return CE_ERR_LAUNCH;
  float* p = g_reduce_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_reduce_scratch_mu);
    p = g_reduce_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(reduce_scratch)) != hipSuccess || addr == nullptr)
        return CE_ERR_LAUNCH;
      p = static_cast<float*>(addr);
      g_reduce_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return CE_OK;
}

}  // namespace

namespace ce_host {
bool take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  if (t_launch_start == nullptr && t_launch_stop == nullptr) return false;
  *start = t_launch_start;
  *stop = t_launch_stop;
  t_launch_start = t_launch_stop = nullptr;
  return true;
}
}  // namespace ce_host

extern "C" {

}  // extern "C"

namespace {

// The row kernels' entry.  op kOpCE: targets and loss_out required;
// grad_out null gives the loss only, grad_out == logits (with equal row
// strides) the gradient in place.  op kOpSoftmax: targets unused; grad_out
// (the softmax) required, or the logits themselves; loss_out (the
// log-sum-exp) may be null.  op kOpShard: targets and loss_out (B records
// of 4 floats, 16-byte aligned) required, grad_out null; col0 is the
// shard's first column.  ldz, ldg: row strides in elements (>= C).  With
// has_ignore (kOpCE only), rows whose target equals ignore are left out of
// the mean: ws (>= 4 bytes, 4-aligned) receives the count of kept rows.
struct FwdArgs {
  int op = ce::kOpCE;
  const void* logits = nullptr;
  int64_t ldz = 0;
  const int32_t* targets = nullptr;
  int64_t B = 0, C = 0;
  int dtype = CE_F32;
  void* grad = nullptr;
  int64_t ldg = 0;
  float* loss = nullptr;
  const float* gmul = nullptr;
  int64_t col0 = 0;
  bool has_ignore = false;
  int32_t ignore = 0;
  void* ws = nullptr;
  size_t ws_bytes = 0;
};

template <typename T>
int fwd_dispatch(int op, int path, const void* z, const int32_t* t, int64_t B, int64_t C, void* g,
                 float* l, ce::RowArgs rs, hipStream_t st, uint64_t* in_place) {
  const T* zz = (const T*)z;
  T* gg = (T*)g;
  switch (op) {
    case ce::kOpCE:
      if (!g) return fwd_typed<T, ce::kOpCE, false>(path, zz, t, B, C, nullptr, l, rs, st);
      return fwd_typed<T, ce::kOpCE, true>(path, zz, t, B, C, gg, l, rs, st, in_place);
    case ce::kOpSoftmax:
      return fwd_typed<T, ce::kOpSoftmax, true>(path, zz, t, B, C, gg, l, rs, st);
    case ce::kOpShard:
      return fwd_typed<T, ce::kOpShard, false>(path, zz, t, B, C, nullptr, l, rs, st);
    default:
      return CE_ERR_PATH;
  }
}

bool known_dtype(int dtype) { return dtype == CE_F32 || dtype == CE_BF16 || dtype == CE_F16; }

// Bytes from the first element of row 0 to the end of row B-1.
uintptr_t span_bytes(int64_t B, int64_t C, int64_t ld, int es) {
  return ((uintptr_t)(B - 1) * (uintptr_t)ld + (uintptr_t)C) * (uintptr_t)es;
}

int fwd_impl(const FwdArgs& a, void* stream) {
  if (!a.logits) return CE_ERR_NULL;
  if (a.op != ce::kOpSoftmax && (!a.targets || !a.loss)) return CE_ERR_NULL;
  if (a.op == ce::kOpSoftmax && !a.grad) return CE_ERR_NULL;
  if (a.has_ignore && !a.ws) return CE_ERR_WORKSPACE;
  if (!known_dtype(a.dtype)) return CE_ERR_DTYPE;
  const int64_t B = a.B, C = a.C;
  if (B <= 0 || C <= 0 || B > 0x7fffffffLL || C > CE_MAX_C) return CE_ERR_SHAPE;
  if (a.ldz < C || (a.grad && a.ldg < C)) return CE_ERR_SHAPE;
  const int es = elem_size(a.dtype);
  const int64_t ldg = a.grad ? a.ldg : a.ldz;
  if ((uint64_t)B > UINT64_MAX / 4 / ((uint64_t)(a.ldz > ldg ? a.ldz : ldg) * es)) return CE_ERR_SHAPE;
  if (a.has_ignore && a.ws_bytes < 4) return CE_ERR_WORKSPACE;
  const uintptr_t z = (uintptr_t)a.logits, g = (uintptr_t)a.grad;
  if (z % es || g % es || (uintptr_t)a.targets % 4) return CE_ERR_ALIGN;
  if ((uintptr_t)a.loss % (a.op == ce::kOpShard ? 16 : 4)) return CE_ERR_ALIGN;
  if (a.gmul && (uintptr_t)a.gmul % 4) return CE_ERR_ALIGN;
  if (a.has_ignore && (uintptr_t)a.ws % 4) return CE_ERR_ALIGN;
  // every row of grad must start at the same offset modulo 16 as its row of
  // logits
  if (a.grad && ((z > g ? z - g : g - z) % 16 || ((a.ldz - ldg) * es) % 16)) return CE_ERR_ALIGN;
  const uintptr_t zspan = span_bytes(B, C, a.ldz, es);
  const bool in_place = a.grad && g == z && ldg == a.ldz;
  if (a.grad && !in_place && overlaps(z, zspan, g, span_bytes(B, C, ldg, es))) return CE_ERR_ALIAS;

  const int forced = g_force_path.load(std::memory_order_relaxed);
  int path = forced ? forced : auto_path(C, es);
  // In place, rows of several parts keep path 4 when the workspace holds
  // their words (in_place_words).
  const bool ip_parts = in_place && a.op == ce::kOpCE && multi_part_row(C, es) &&
                        in_place_words(a.ws, a.ws_bytes, B) != nullptr;
  if (!a.grad || in_place) {
    if (path == kPathParts && (!a.grad || (multi_part_row(C, es) && !ip_parts))) {
      if (forced) return CE_ERR_PATH;
      path = path_without_parts(C, es, a.grad != nullptr);
    }
  }
  uint64_t* const ip_words =
      ip_parts && path == kPathParts ? in_place_words(a.ws, a.ws_bytes, B) : nullptr;
  const bool short_ok = short_span_ok(C, a.ldz, es) && (!a.grad || short_span_ok(C, ldg, es));
  if (path == kPathShort && !forced && !short_ok) path = kPathResident;
  // path 5 loads vectors that every row start of both arrays is aligned to
  // and that divide the row length and strides; rows it has no
  // configuration for run on path 2
  int wave_vb = 0;
  if (path == kPathWave) {
    const int64_t lens = C | a.ldz | (a.grad ? ldg : 0);
    wave_vb = short_vw(lens, es, z, a.grad ? g : 0, 16 / es) * es;
    if (ce_wave::lane_bytes(C, es, wave_vb) == 0) {
      if (forced) return CE_ERR_PATH;
      path = kPathResident;
    }
  }
  // a forced path that cannot take the shape is refused before any launch
  bool takes = false;
  switch (path) {
    case kPathShort: takes = short_ok; break;
    case kPathResident: resident_cfg(C, es, &takes); break;
    case kPathLong: takes = true; break;
    case kPathParts: takes = a.grad && body_vectors_max(C, es) <= parts_max(es); break;
    case kPathWave: takes = true; break;
    default: break;
  }
  if (!takes) return CE_ERR_PATH;
  const hipStream_t st = as_stream(stream);
  ce::RowArgs rs{1.0f / (float)B, a.gmul, a.col0, a.ldz, ldg, nullptr, a.ignore,
                 a.has_ignore ? 1 : 0};
  if (a.has_ignore) {
    uint32_t* kept = (uint32_t*)a.ws;
    const int64_t rounds = (B + ce::kCountRound - 1) / ce::kCountRound;
    if (B <= kCountOneRows) {
      ce_host::launch(ce::ce_count_kept_kernel<true>, dim3(1), dim3(ce::kCountThreads), 0, st,
                      a.targets, B, a.ignore, kept);
    } else {
      ce_host::launch(ce::ce_set_u32_kernel, dim3(1), dim3(64), 0, st, kept, 0u);
      if (launched() != CE_OK) return CE_ERR_LAUNCH;
      ce_host::launch(ce::ce_count_kept_kernel<false>,
                      dim3((unsigned)(rounds < kCountMaxBlocks ? rounds : kCountMaxBlocks)),
                      dim3(ce::kCountThreads), 0, st, a.targets, B, a.ignore, kept);
    }
    if (launched() != CE_OK) return CE_ERR_LAUNCH;
    rs.kept = kept;
  }
  if (path == kPathWave)
    return ce_wave::launch(a.dtype, a.op, a.grad != nullptr, wave_vb, a.logits, a.targets, B,
                           (int)C, rs, a.grad, a.loss, st);
  switch (a.dtype) {
    case CE_F32:
      return fwd_dispatch<float>(a.op, path, a.logits, a.targets, B, C, a.grad, a.loss, rs, st,
                                 ip_words);
    case CE_BF16:
      return fwd_dispatch<__bf16>(a.op, path, a.logits, a.targets, B, C, a.grad, a.loss, rs, st,
                                  ip_words);
    default:
      return fwd_dispatch<_Float16>(a.op, path, a.logits, a.targets, B, C, a.grad, a.loss, rs, st,
                                    ip_words);
  }
}

// The contiguous calls.
int fwd_plain(int op, const void* logits, const int32_t* targets, int64_t B, int64_t C, int dtype,
              void* grad_out, float* loss_out, const float* gmul, int64_t col0, void* stream) {
  FwdArgs a;
  a.op = op;
  a.logits = logits;
  a.ldz = C;
  a.targets = targets;
  a.B = B;
  a.C = C;
  a.dtype = dtype;
  a.grad = grad_out;
  a.ldg = C;
  a.loss = loss_out;
  a.gmul = gmul;
  a.col0 = col0;
  return fwd_impl(a, stream);
}

template <typename T>
int launch_scale(T* g, int64_t n, const float* scale, hipStream_t st) {
  constexpr int64_t chunk = (int64_t)ce::kScaleThreads * ce::kScaleSlots;
  const int64_t nb = n / (16 / (int64_t)sizeof(T)) + 1;
  const int64_t blocks = (nb + chunk - 1) / chunk;
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  ce_host::launch(ce::ce_scale_kernel<T>, dim3((unsigned)blocks), dim3(ce::kScaleThreads), 0, st,
                     g, n, scale);
  return launched();
}

// ------------------------------------------------------- softmax backward
// Row configurations that hold both y and dy of a row in registers (NT
// threads x NV 16-byte vectors of each); longer rows stream the rest.
constexpr RowCfg kBwdCfgs[] = {{64, 1},   {64, 2},   {64, 4},   {256, 2},
                               {256, 4},  {1024, 2}, {1024, 4}, {1024, 8}};
constexpr RowCfg kBwdLongCfg = {1024, 8};
constexpr RowCfg kBwdLongTestCfg = {256, 1};

template <typename T, int S, int EPL, int VW>
int launch_bwd_short_cfg(const T* y, const T* dy, int64_t B, int C, T* dx, hipStream_t st) {
  constexpr int rpb = ce::kShortThreads / S;
  const int64_t blocks = (B + rpb - 1) / rpb;
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  ce_host::launch((ce::sm_bwd_short_kernel<T, S, EPL, VW>), dim3((unsigned)blocks),
                     dim3(ce::kShortThreads), 0, st, y, dy, B, C, dx);
  return launched();
}

template <typename T, int S, int EPL>
int launch_bwd_short_vw(int vw, const T* y, const T* dy, int64_t B, int C, T* dx, hipStream_t st) {
  switch (vw) {
    case 1: return launch_bwd_short_cfg<T, S, EPL, 1>(y, dy, B, C, dx, st);
    case 2: return launch_bwd_short_cfg<T, S, EPL, 2>(y, dy, B, C, dx, st);
    case 4: return launch_bwd_short_cfg<T, S, EPL, 4>(y, dy, B, C, dx, st);
    case 8:
      if constexpr (sizeof(T) == 2 && EPL >= 8) return launch_bwd_short_cfg<T, S, EPL, 8>(y, dy, B, C, dx, st);
      return CE_ERR_PATH;
    default: return CE_ERR_PATH;
  }
}

// Rows of more than 64 bytes that 16-byte vectors do not divide, with y (and
// so dy and dx, congruent to it) 16-byte aligned: the LDS-staged backward.
// S is the smallest of 8, 16 and 32 whose 16 slots cover the row and whose
// pass of 256/S rows fits half a staged chunk; EPL is 8, 12 or 16.
bool staged_bwd_rows(const void* y, int64_t C, int es) {
  return C * es > ce::kTinyRowBytes && (C * es) % 16 != 0 && (uintptr_t)y % 16 == 0 &&
         staged_bwd_lanes(C, es) > 0;
}

template <typename T, int S, int EPL>
int launch_bwd_staged_cfg(const T* y, const T* dy, int64_t B, int64_t C, T* dx, hipStream_t st) {
  auto kern = ce::sm_bwd_staged_kernel<T, S, EPL>;
  static std::atomic<int> occupancy{0};
  const int res = resident_blocks(reinterpret_cast<const void*>(kern), ce::kStagedThreads, occupancy);
  if (res < 1) return CE_ERR_LAUNCH;
  const int64_t rows = ce::staged_rows_per_chunk((int)C, (int)sizeof(T), ce::kStagedThreads / S,
                                                 ce::kStagedBwdChunkBytes);
  if (rows < 1 || C > S * EPL) return CE_ERR_PATH;
  const int64_t chunks = (B + rows - 1) / rows;
  const int64_t grid = chunks < res ? chunks : res;
  ce_host::launch(kern, dim3((unsigned)grid), dim3(ce::kStagedThreads), 0, st, y, dy, B, (int)C,
                     dx);
  return launched();
}

template <typename T, int S>
int launch_bwd_staged_s(const T* y, const T* dy, int64_t B, int64_t C, T* dx, hipStream_t st) {
  if (C <= 8 * S) return launch_bwd_staged_cfg<T, S, 8>(y, dy, B, C, dx, st);
  if (C <= 12 * S) return launch_bwd_staged_cfg<T, S, 12>(y, dy, B, C, dx, st);
  return launch_bwd_staged_cfg<T, S, 16>(y, dy, B, C, dx, st);
}

template <typename T>
int launch_bwd_staged(const T* y, const T* dy, int64_t B, int64_t C, T* dx, hipStream_t st) {
  switch (staged_bwd_lanes(C, sizeof(T))) {
    case 8: return launch_bwd_staged_s<T, 8>(y, dy, B, C, dx, st);
    case 16: return launch_bwd_staged_s<T, 16>(y, dy, B, C, dx, st);
    case 32: return launch_bwd_staged_s<T, 32>(y, dy, B, C, dx, st);
    default: return CE_ERR_PATH;
  }
}

// The short layout of the loss (S lanes per row, about 16 bytes of each
// array per lane), with a vector width that all three arrays' rows allow.
template <typename T>
int launch_bwd_short(const T* y, const T* dy, int64_t B, int64_t C, T* dx, hipStream_t st) {
  if (C > kShortMaxC) return CE_ERR_PATH;
  constexpr int es = sizeof(T);
  constexpr int E16 = 16 / es;
  const int c = (int)C;
  const uintptr_t other = (uintptr_t)dy | (uintptr_t)dx;  // aligned iff both are
  auto vw = [&](int epl) { return short_vw(C, es, (uintptr_t)y, other, epl); };
  if (C <= E16) return launch_bwd_short_vw<T, 1, E16>(vw(E16), y, dy, B, c, dx, st);
  if (C <= 2 * E16) return launch_bwd_short_vw<T, 2, E16>(vw(E16), y, dy, B, c, dx, st);
  if (C <= 4 * E16) return launch_bwd_short_vw<T, 4, E16>(vw(E16), y, dy, B, c, dx, st);
  if (C <= 8 * E16) return launch_bwd_short_vw<T, 8, E16>(vw(E16), y, dy, B, c, dx, st);
  if (C <= 16 * E16) return launch_bwd_short_vw<T, 16, E16>(vw(E16), y, dy, B, c, dx, st);
  if constexpr (E16 < 16) {
    if (C <= 32 * E16) return launch_bwd_short_vw<T, 16, 2 * E16>(vw(2 * E16), y, dy, B, c, dx, st);
  }
  if constexpr (E16 < 8) {
    if (C <= 64 * E16) return launch_bwd_short_vw<T, 16, 4 * E16>(vw(4 * E16), y, dy, B, c, dx, st);
  }
  return CE_ERR_PATH;
}

template <typename T, int NT, int NV>
int launch_bwd_row_cfg(const T* y, const T* dy, int64_t B, int64_t C, T* dx, hipStream_t st) {
  auto kern = ce::sm_bwd_row_kernel<T, NT, NV>;
  static std::atomic<int> occupancy{0};
  const int res = resident_blocks(reinterpret_cast<const void*>(kern), NT, occupancy);
  if (res < 1) return CE_ERR_LAUNCH;
  const int64_t grid = B < res ? B : res;
  ce_host::launch(kern, dim3((unsigned)grid), dim3(NT), 0, st, y, dy, B, (int)C, dx);
  return launched();
}

template <typename T>
int launch_bwd_row(RowCfg cfg, const T* y, const T* dy, int64_t B, int64_t C, T* dx, hipStream_t st) {
#define CE_BWD_CASE(NT_, NV_) \
  if (cfg.nt == NT_ && cfg.nv == NV_) return launch_bwd_row_cfg<T, NT_, NV_>(y, dy, B, C, dx, st);
  CE_BWD_CASE(64, 1)
  CE_BWD_CASE(64, 2)
  CE_BWD_CASE(64, 4)
  CE_BWD_CASE(256, 1)
  CE_BWD_CASE(256, 2)
  CE_BWD_CASE(256, 4)
  CE_BWD_CASE(1024, 2)
  CE_BWD_CASE(1024, 4)
  CE_BWD_CASE(1024, 8)
#undef CE_BWD_CASE
  return CE_ERR_PATH;
}

// Row parts of the backward: four parts of four register slots of y and of
// dy (1024 threads) for bodies of up to 16384 16-byte vectors per array
// (bf16 C up to 131072, fp32 C up to 65536), eight such parts up to 32768
// (bf16 C up to 262144, fp32 C up to 131072); out of place only (a part's
// mailbox is in dx and a recompute reads its partner's y and dy).
constexpr int kBwdPartSlots = 4;
constexpr int64_t kBwdPartsFour = (int64_t)4 * kBwdPartSlots * 1024;
constexpr int64_t kBwdPartsMax = (int64_t)8 * kBwdPartSlots * 1024;
constexpr int64_t kBwdPartsMin = 128;  // every part keeps at least its two mailbox vectors

bool bwd_parts_take(int64_t C, int es, bool in_place) {
  const int64_t nb = body_vectors_max(C, es);
  return !in_place && nb >= kBwdPartsMin && nb <= kBwdPartsMax;
}

int bwd_auto_path(int64_t C, int es, bool in_place) {
  if (C <= kShortMaxC) return kPathShort;
  if (ce_wave::bwd_lane_bytes(C, es, wave_vb_contiguous(C, es)) != 0) return kPathWave;
  if (row_vectors(C, es) <= (int64_t)kBwdLongCfg.nt * kBwdLongCfg.nv) return kPathResident;
  if (bwd_parts_take(C, es, in_place)) return kPathParts;
  return kPathLong;
}

template <typename T, int P>
int launch_bwd_parts_p(const T* y, const T* dy, int64_t B, int64_t C, T* dx, hipStream_t st) {
  const int64_t blocks = P * ((B + 7) / 8 * 8);
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  ce_host::launch((ce::sm_bwd_part_kernel<T, P, 1024, kBwdPartSlots>), dim3((unsigned)blocks),
                     dim3(1024), 0, st, y, dy, B, (int)C, dx,
                     g_part_polls.load(std::memory_order_relaxed),
                     g_part_counter.load(std::memory_order_relaxed));
  return launched();
}

template <typename T>
int launch_bwd_parts(const T* y, const T* dy, int64_t B, int64_t C, T* dx, hipStream_t st) {
  if (body_vectors_max(C, sizeof(T)) <= kBwdPartsFour)
    return launch_bwd_parts_p<T, 4>(y, dy, B, C, dx, st);
  return launch_bwd_parts_p<T, 8>(y, dy, B, C, dx, st);
}

template <typename T>
int softmax_bwd_typed(int path, const T* y, const T* dy, int64_t B, int64_t C, T* dx,
                      bool in_place, hipStream_t st) {
  const bool forced = g_force_path.load(std::memory_order_relaxed) != 0;
  switch (path) {
    case kPathParts:
      if (!bwd_parts_take(C, sizeof(T), in_place)) return CE_ERR_PATH;
      return launch_bwd_parts<T>(y, dy, B, C, dx, st);
    case kPathShort:
      if (!forced && staged_bwd_rows(y, C, sizeof(T)))
        return launch_bwd_staged<T>(y, dy, B, C, dx, st);
      return launch_bwd_short<T>(y, dy, B, C, dx, st);
    case kPathResident: {
      if constexpr (sizeof(T) == 2) {
        if (!forced && staged_bwd_rows(y, C, sizeof(T)))
          return launch_bwd_staged<T>(y, dy, B, C, dx, st);
      }
      const bool aligned = (uintptr_t)y % 16 == 0 && (C * sizeof(T)) % 16 == 0;  // dy, dx: congruent
      const int64_t need = row_need(C, sizeof(T), aligned);
      for (const RowCfg& r : kBwdCfgs)
        if ((int64_t)r.nt * r.nv >= need) return launch_bwd_row<T>(r, y, dy, B, C, dx, st);
      return CE_ERR_PATH;
    }
    case kPathLong:
      return launch_bwd_row<T>(forced ? kBwdLongTestCfg : kBwdLongCfg, y, dy, B, C, dx, st);
    default:
      return CE_ERR_PATH;
  }
}

// --------------------------------------------------------- vocabulary shards
constexpr int kMaxShards = 1024;

template <typename T>
int launch_shard_grad(const T* z, const int32_t* t, int64_t B, int64_t C, int64_t col0,
                      int64_t Ctot, const float* recs, int nshards, ce::RowArgs rs, T* g,
                      float* l, hipStream_t st) {
  const ce::f32x4* r4 = reinterpret_cast<const ce::f32x4*>(recs);
  if (C <= ce::kShardTinyC) {
    const int64_t blocks = (B + 255) / 256;
    if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
    ce_host::launch(ce::ce_shard_grad_tiny_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st,
                       z, t, B, (int)C, col0, Ctot, r4, nshards, rs, g, l);
    return launched();
  }
  // units of one wave x 8 slots for rows of at most 512 vectors, else of
  // four waves x 2 slots
  const int64_t nb = body_vectors_max(C, sizeof(T));
  const bool wave_units = nb <= 64 * 8;
  const int64_t chunk = wave_units ? 64 * 8 : 256 * 2;
  const int64_t units = ce::kShardThreads / (wave_units ? 64 : 256);
  const int64_t chunks = nb > 0 ? (nb + chunk - 1) / chunk : 1;
  const int64_t blocks = (B * chunks + units - 1) / units;
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  if (wave_units)
    ce_host::launch((ce::ce_shard_grad_kernel<T, 64, 8>), dim3((unsigned)blocks),
                       dim3(ce::kShardThreads), 0, st, z, t, B, (int)C, col0, Ctot, r4, nshards, rs,
                       g, l, (int)chunks);
  else
    ce_host::launch((ce::ce_shard_grad_kernel<T, 256, 2>), dim3((unsigned)blocks),
                       dim3(ce::kShardThreads), 0, st, z, t, B, (int)C, col0, Ctot, r4, nshards, rs,
                       g, l, (int)chunks);
  return launched();
}

int launch_reduce(const float* rows, int64_t B, float* out, float* part, hipStream_t st) {
  const int64_t blocks = reduce_blocks(B);
  if (blocks == 1) {
    ce_host::launch(ce::ce_reduce_one_kernel, dim3(1), dim3(ce::kReduceOneThreads), 0, st, rows,
                    (int)B, out);
    return launched();
  }
  ce_host::launch(ce::ce_reduce_kernel, dim3((unsigned)blocks), dim3(ce::kReduceThreads), 0, st,
                  rows, B, reduce_chunk(B), part);
  if (launched() != CE_OK) return CE_ERR_LAUNCH;
  ce_host::launch(ce::ce_reduce_one_kernel, dim3(1), dim3(ce::kReduceOneThreads), 0, st,
                  (const float*)part, (int)blocks, out);
  return launched();
}

}  // namespace

extern "C" {

int ce_fwd_grad(const void* logits, const int32_t* targets, int64_t B, int64_t C, int dtype,
                void* grad_out, float* loss_out, void* stream) {
  if (!grad_out) return CE_ERR_NULL;
  return fwd_plain(ce::kOpCE, logits, targets, B, C, dtype, grad_out, loss_out, nullptr, 0, stream);
}

int ce_fwd_loss(const void* logits, const int32_t* targets, int64_t B, int64_t C, int dtype,
                float* loss_out, void* stream) {
  return fwd_plain(ce::kOpCE, logits, targets, B, C, dtype, nullptr, loss_out, nullptr, 0, stream);
}

int ce_fwd_grad_scaled(const void* logits, const int32_t* targets, int64_t B, int64_t C,
                       int dtype, void* grad_out, float* loss_out, const float* grad_scale,
                       void* stream) {
  if (!grad_scale || !grad_out) return CE_ERR_NULL;
  return fwd_plain(ce::kOpCE, logits, targets, B, C, dtype, grad_out, loss_out, grad_scale, 0,
                   stream);
}

size_t ce_fwd_workspace_bytes(int32_t ignore_index) {
  return ignore_index == CE_NO_IGNORE ? 0 : 4;
}

size_t ce_fwd_inplace_workspace_bytes(int64_t B) {
  if (B <= 0 || B > 0x7fffffffLL) return 0;
  return kInPlaceWordsOffset + (size_t)B * kInPlaceRowBytes;
}

int ce_fwd_grad_ex(const void* logits, int64_t ld_logits, const int32_t* targets, int64_t B,
                   int64_t C, int dtype, void* grad_out, int64_t ld_grad, float* loss_out,
                   const float* grad_scale, int32_t ignore_index, void* workspace,
                   size_t workspace_bytes, void* stream) {
  FwdArgs a;
  a.logits = logits;
  a.ldz = ld_logits;
  a.targets = targets;
  a.B = B;
  a.C = C;
  a.dtype = dtype;
  a.grad = grad_out;
  a.ldg = ld_grad;
  a.loss = loss_out;
  a.gmul = grad_scale;
  a.has_ignore = ignore_index != CE_NO_IGNORE;
  a.ignore = ignore_index;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  return fwd_impl(a, stream);
}

int ce_scale_grad(void* grad, int64_t n, int dtype, const float* scale, void* stream) {
  if (!grad || !scale) return CE_ERR_NULL;
  if (!known_dtype(dtype)) return CE_ERR_DTYPE;
  if (n <= 0) return CE_ERR_SHAPE;
  const int es = elem_size(dtype);
  if ((uintptr_t)grad % es || (uintptr_t)scale % 4) return CE_ERR_ALIGN;
  if ((uint64_t)n > UINT64_MAX / 2 / (uint64_t)es) return CE_ERR_SHAPE;
  if (overlaps((uintptr_t)grad, (uintptr_t)n * es, (uintptr_t)scale, 4)) return CE_ERR_ALIAS;
  const hipStream_t st = as_stream(stream);
  if (dtype == CE_F32) return launch_scale<float>((float*)grad, n, scale, st);
  if (dtype == CE_BF16) return launch_scale<__bf16>((__bf16*)grad, n, scale, st);
  return launch_scale<_Float16>((_Float16*)grad, n, scale, st);
}

int ce_softmax_fwd(const void* x, int64_t B, int64_t C, int dtype, void* y_out, float* lse_out,
                   void* stream) {
  return fwd_plain(ce::kOpSoftmax, x, nullptr, B, C, dtype, y_out, lse_out, nullptr, 0, stream);
}

int ce_softmax_bwd(const void* y, const void* dy, int64_t B, int64_t C, int dtype, void* dx_out,
                   void* stream) {
  if (!y || !dy || !dx_out) return CE_ERR_NULL;
  if (!known_dtype(dtype)) return CE_ERR_DTYPE;
  if (B <= 0 || C <= 0 || B > 0x7fffffffLL || C > CE_MAX_C) return CE_ERR_SHAPE;
  const int es = elem_size(dtype);
  const uintptr_t a = (uintptr_t)y, b = (uintptr_t)dy, o = (uintptr_t)dx_out;
  if (a % es || b % es || o % es) return CE_ERR_ALIGN;
  if ((a > b ? a - b : b - a) % 16 || (a > o ? a - o : o - a) % 16) return CE_ERR_ALIGN;
  if ((uint64_t)B > UINT64_MAX / ((uint64_t)C * es)) return CE_ERR_SHAPE;
  const uintptr_t n = (uintptr_t)B * (uintptr_t)C * es;
  // dx may be y or dy themselves (every element is read before the thread
  // that reads it writes it), but no other overlap
  if (o != a && overlaps(o, n, a, n)) return CE_ERR_ALIAS;
  if (o != b && overlaps(o, n, b, n)) return CE_ERR_ALIAS;
  const bool in_place = o == a || o == b;
  const int forced = g_force_path.load(std::memory_order_relaxed);
  int path = forced ? forced : bwd_auto_path(C, es, in_place);
  const hipStream_t st = as_stream(stream);
  if (path == kPathWave) {
    // y, dy and dx are congruent modulo 16 bytes: y's alignment serves all
    const int vb = short_vw(C, es, a, 0, 16 / es) * es;
    if (ce_wave::bwd_lane_bytes(C, es, vb) != 0)
      return ce_wave::launch_bwd(dtype, vb, y, dy, B, (int)C, dx_out, st);
    if (forced) return CE_ERR_PATH;
    path = kPathResident;
  }
  if (dtype == CE_F32)
    return softmax_bwd_typed<float>(path, (const float*)y, (const float*)dy, B, C, (float*)dx_out,
                                    in_place, st);
  if (dtype == CE_BF16)
    return softmax_bwd_typed<__bf16>(path, (const __bf16*)y, (const __bf16*)dy, B, C,
                                     (__bf16*)dx_out, in_place, st);
  return softmax_bwd_typed<_Float16>(path, (const _Float16*)y, (const _Float16*)dy, B, C,
                                     (_Float16*)dx_out, in_place, st);
}

int ce_shard_stats(const void* logits, const int32_t* targets, int64_t B, int64_t C, int64_t col0,
                   int dtype, float* records_out, void* stream) {
  if (col0 < 0 || col0 > 0x7fffffffLL) return CE_ERR_SHAPE;
  return fwd_plain(ce::kOpShard, logits, targets, B, C, dtype, nullptr, records_out, nullptr, col0,
                   stream);
}

int ce_shard_grad(const void* logits, const int32_t* targets, int64_t B, int64_t C, int64_t col0,
                  int64_t C_total, int dtype, const float* records, int n_shards, void* grad_out,
                  float* loss_out, const float* grad_scale, void* stream) {
  if (!logits || !targets || !records || !grad_out) return CE_ERR_NULL;
  if (!known_dtype(dtype)) return CE_ERR_DTYPE;
  if (B <= 0 || C <= 0 || B > 0x7fffffffLL || C > CE_MAX_C) return CE_ERR_SHAPE;
  if (n_shards < 1 || n_shards > kMaxShards) return CE_ERR_SHAPE;
  if (col0 < 0 || C_total < C || col0 > C_total - C || C_total > 0x7fffffffLL) return CE_ERR_SHAPE;
  const int es = elem_size(dtype);
  const uintptr_t z = (uintptr_t)logits, g = (uintptr_t)grad_out;
  if (z % es || g % es || (uintptr_t)targets % 4 || (uintptr_t)records % 16) return CE_ERR_ALIGN;
  if ((uintptr_t)loss_out % 4 || (uintptr_t)grad_scale % 4) return CE_ERR_ALIGN;
  if ((z > g ? z - g : g - z) % 16) return CE_ERR_ALIGN;
  if ((uint64_t)B > UINT64_MAX / ((uint64_t)C * es)) return CE_ERR_SHAPE;
  const uintptr_t n = (uintptr_t)B * (uintptr_t)C * es;
  if (g != z && overlaps(z, n, g, n)) return CE_ERR_ALIAS;
  if (overlaps(g, n, (uintptr_t)records, (uintptr_t)n_shards * (uintptr_t)B * 16)) return CE_ERR_ALIAS;
  const ce::RowArgs rs{1.0f / (float)B, grad_scale, col0, C, C, nullptr, 0, 0};
  const hipStream_t st = as_stream(stream);
  if (dtype == CE_F32)
    return launch_shard_grad<float>((const float*)logits, targets, B, C, col0, C_total, records,
                                    n_shards, rs, (float*)grad_out, loss_out, st);
  if (dtype == CE_BF16)
    return launch_shard_grad<__bf16>((const __bf16*)logits, targets, B, C, col0, C_total, records,
                                     n_shards, rs, (__bf16*)grad_out, loss_out, st);
  return launch_shard_grad<_Float16>((const _Float16*)logits, targets, B, C, col0, C_total,
                                     records, n_shards, rs, (_Float16*)grad_out, loss_out, st);
}

size_t ce_reduce_workspace_bytes(int64_t B) {
  if (B <= 0 || B > kReduceMaxRows) return 0;
  const int64_t blocks = reduce_blocks(B);
  return blocks > 1 ? (size_t)blocks * sizeof(float) : 0;
}

int ce_reduce_loss(const float* loss_rows, int64_t B, float* loss_scalar_out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!loss_rows || !loss_scalar_out) return CE_ERR_NULL;
  if (B <= 0 || B > kReduceMaxRows) return CE_ERR_SHAPE;
  if ((uintptr_t)loss_rows % 4 || (uintptr_t)loss_scalar_out % 4) return CE_ERR_ALIGN;
  const size_t need = ce_reduce_workspace_bytes(B);
  if (need && (!workspace || workspace_bytes < need)) return CE_ERR_WORKSPACE;
  if (need && (uintptr_t)workspace % 4) return CE_ERR_ALIGN;
  return launch_reduce(loss_rows, B, loss_scalar_out, (float*)workspace, as_stream(stream));
}

int ce_fwd_grad_loss(const void* logits, const int32_t* targets, int64_t B, int64_t C, int dtype,
                     void* grad_out, float* loss_rows_out, float* loss_scalar_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  // the reduction's arguments first: ce_fwd_grad launches once its own
  // arguments pass, and nothing may be launched when the call fails
  if (!loss_scalar_out) return CE_ERR_NULL;
  if ((uintptr_t)loss_scalar_out % 4) return CE_ERR_ALIGN;
  if (B > 0 && B <= kReduceMaxRows) {
    const size_t need = ce_reduce_workspace_bytes(B);
    if (need && (!workspace || workspace_bytes < need)) return CE_ERR_WORKSPACE;
    if (need && (uintptr_t)workspace % 4) return CE_ERR_ALIGN;
  }
  const int st = ce_fwd_grad(logits, targets, B, C, dtype, grad_out, loss_rows_out, stream);
  if (st != CE_OK) return st;
  return ce_reduce_loss(loss_rows_out, B, loss_scalar_out, workspace, workspace_bytes, stream);
}

int ce_reduce_loss_noalloc(const float* loss_rows, int64_t B, float* loss_scalar_out,
                           void* stream) {
  if (!loss_rows || !loss_scalar_out) return CE_ERR_NULL;
  if (B <= 0 || B > CE_NOALLOC_MAX_ROWS) return CE_ERR_SHAPE;
  if ((uintptr_t)loss_rows % 4 || (uintptr_t)loss_scalar_out % 4) return CE_ERR_ALIGN;
  float* part = nullptr;
  static_assert(CE_NOALLOC_MAX_ROWS <= kReduceMaxRows, "noalloc range within the tree's");
  if (reduce_blocks(B) > 1) {
    if (reduce_blocks(B) > kReduceMaxBlocks) return CE_ERR_SHAPE;
    const int rc = reduce_scratch_ptr(&part);
    if (rc != CE_OK) return rc;
  }
  return launch_reduce(loss_rows, B, loss_scalar_out, part, as_stream(stream));
}

const char* ce_status_string(int status) {
  switch (status) {
    case CE_OK: return "ok";
    case CE_ERR_NULL: return "a required pointer is NULL";
    case CE_ERR_SHAPE: return "invalid shape (B and C must be positive and within limits)";
    case CE_ERR_DTYPE: return "unknown dtype";
    case CE_ERR_WORKSPACE: return "workspace missing or too small";
    case CE_ERR_LAUNCH: return "kernel launch failed";
    case CE_ERR_ALIGN: return "pointer alignment not supported";
    case CE_ERR_ALIAS: return "an output overlaps an input in a way the call refuses";
    case CE_ERR_PATH: return "the forced kernel path cannot take this shape";
    default: return "unknown status";
  }
}

const char* ce_version(void) { return "ce_mi355x 0.1.0 gfx950"; }

int ce_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst) return CE_ERR_NULL;
  if (bytes <= 0 || bytes % 16) return CE_ERR_SHAPE;
  if ((uintptr_t)src % 16 || (uintptr_t)dst % 16) return CE_ERR_ALIGN;
  if (overlaps((uintptr_t)src, (uintptr_t)bytes, (uintptr_t)dst, (uintptr_t)bytes)) return CE_ERR_ALIAS;
  const int64_t blocks = (bytes + ce::kCopyChunk - 1) / ce::kCopyChunk;
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  ce_host::launch(ce::ce_copy_kernel, dim3((unsigned)blocks), dim3(ce::kCopyThreads), 0,
                     as_stream(stream), (const char*)src, (char*)dst, bytes);
  return launched();
}

int ce_select_path(int64_t C, int dtype) {
  if (!known_dtype(dtype)) return CE_ERR_DTYPE;
  if (C <= 0 || C > CE_MAX_C) return CE_ERR_SHAPE;
  const int forced = g_force_path.load(std::memory_order_relaxed);
  return forced ? forced : auto_path(C, elem_size(dtype));
}

int ce_debug_force_path(int path) {
  if (path < 0 || path > kPathWave) return CE_ERR_PATH;
  return g_force_path.exchange(path);
}

int ce_debug_part_polls(int polls) {
  if (polls < 0) return CE_ERR_PATH;
  return g_part_polls.exchange(polls);
}

int ce_debug_time_next_launch(void* start_event, void* stop_event) {
  t_launch_start = static_cast<hipEvent_t>(start_event);
  t_launch_stop = static_cast<hipEvent_t>(stop_event);
  return CE_OK;
}

int ce_debug_part_counter(uint32_t* device_counter) {
  g_part_counter.store(device_counter);
  return CE_OK;
}

}  // extern "C"
