// Device-side building blocks for the gfx950 cross-entropy kernels:
// element traits (fp32 / bf16 in 16-byte vectors), buffer-resource memory
// access with hardware range checks, and cross-lane reductions over DPP and
// ds_swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ce {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Reinterpret whole vectors only.  With this compiler, __builtin_bit_cast of
// a single component (e.g. bit_cast<float>(v.y)) reads component 0, so
// component bit casts are never written.
__device__ __forceinline__ f32x4 as_f32(u32x4 v) { return __builtin_bit_cast(f32x4, v); }
__device__ __forceinline__ f32x2 as_f32(u32x2 v) { return __builtin_bit_cast(f32x2, v); }
__device__ __forceinline__ u32x4 as_u32(f32x4 v) { return __builtin_bit_cast(u32x4, v); }
__device__ __forceinline__ u32x2 as_u32(f32x2 v) { return __builtin_bit_cast(u32x2, v); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// log2(e) and ln(2) rounded to float32.  Exponentials are evaluated as
// exp2(x * log2(e)) on the hardware v_exp_f32, logarithms as v_log_f32.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLowest = -3.402823466e38f;  // finite start value of a running max

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
// Maxima as IEEE maximum (a NaN operand gives NaN; -0 < +0): one
// v_maximum3_f32, where fmaxf would first quiet each operand that is not
// the result of arithmetic (a load, a DPP move) with an extra v_max.
__device__ __forceinline__ float fmax2(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmax2(fmax2(a, b), c); }

// ---------------------------------------------------------------------------
// Buffer resources.  A raw buffer access whose byte offset is at or beyond
// num_records returns zero (loads) or is dropped (stores) in hardware, so a
// resource sized to exactly the valid bytes of a row makes the row's edge
// free of bounds branches.  Third-word value: the gfx9 buffer format word.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
// cache-policy operand of the buffer builtins: bit 1 = nt (streaming, do
// not keep in the caches)
constexpr int kPolicyStream = 2;
constexpr int kPolicyDefault = 0;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

template <int POLICY>
__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, POLICY);
}
// A store wider than 8 bytes reads its data registers after it issues; a
// VALU write to those registers in the next two wait states corrupts the
// stored data.  The compiler inserts those wait states only when soffset is
// not a register, so every 16-byte store here is followed by them
// explicitly, with nothing scheduled in between.
__device__ __forceinline__ void wide_store_guard() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);
}

template <int POLICY>
__device__ __forceinline__ void bstore128(u32x4 v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, POLICY);
  wide_store_guard();
}

// ---------------------------------------------------------------------------
// Element traits.  A 16-byte vector holds VE elements; unpack widens them
// to float32 (bf16 -> f32 is exact: the bf16 bits become the high half;
// f16 -> f32 is exact too), pack rounds float32 back (bf16:
// v_cvt_pk_bf16_f32, f16: v_cvt_f16_f32; both nearest-even).
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int VE = 4;
  static constexpr unsigned kNegInfWord = 0xFF800000u;  // a 32-bit word of -inf elements
  __device__ static __forceinline__ void unpack(u32x4 v, float (&f)[4]) {
    const f32x4 x = as_f32(v);
    f[0] = x.x;
    f[1] = x.y;
    f[2] = x.z;
    f[3] = x.w;
  }
  __device__ static __forceinline__ u32x4 pack(const float (&g)[4]) {
    return as_u32(f32x4{g[0], g[1], g[2], g[3]});
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ void store1(float* p, float g) {
    __builtin_nontemporal_store(g, p);
  }
  // the vector with element j (0..3) replaced by -inf
  __device__ static __forceinline__ u32x4 kill(u32x4 v, int j) {
    constexpr unsigned kNinf = 0xFF800000u;
    return u32x4{j == 0 ? kNinf : v.x, j == 1 ? kNinf : v.y, j == 2 ? kNinf : v.z,
                 j == 3 ? kNinf : v.w};
  }
};

__device__ __forceinline__ float bf16lo(unsigned d) { return __builtin_bit_cast(float, d << 16); }
__device__ __forceinline__ float bf16hi(unsigned d) {
  return __builtin_bit_cast(float, d & 0xffff0000u);
}
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

template <>
struct Elem<__bf16> {
  static constexpr int VE = 8;
  static constexpr unsigned kNegInfWord = 0xFF80FF80u;
  __device__ static __forceinline__ void unpack(u32x4 v, float (&f)[8]) {
    f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
    f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
    f[4] = bf16lo(v.z); f[5] = bf16hi(v.z);
    f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
  }
  __device__ static __forceinline__ u32x4 pack(const float (&g)[8]) {
    return u32x4{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                 pack_bf16x2(g[6], g[7])};
  }
  __device__ static __forceinline__ float load1(const __bf16* p) {
    unsigned short h = *reinterpret_cast<const unsigned short*>(p);
    return __builtin_bit_cast(float, (unsigned)h << 16);
  }
  __device__ static __forceinline__ void store1(__bf16* p, float g) {
    unsigned d = pack_bf16x2(g, 0.f);
    __builtin_nontemporal_store((unsigned short)(d & 0xffffu),
                                reinterpret_cast<unsigned short*>(p));
  }
  // the vector with element j (0..7) replaced by -inf (bf16 0xFF80)
  __device__ static __forceinline__ u32x4 kill(u32x4 v, int j) {
    const int d = j >> 1;
    const unsigned keep = (j & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    const unsigned ninf = (j & 1) ? 0xFF800000u : 0x0000FF80u;
    return u32x4{d == 0 ? (v.x & keep) | ninf : v.x, d == 1 ? (v.y & keep) | ninf : v.y,
                 d == 2 ? (v.z & keep) | ninf : v.z, d == 3 ? (v.w & keep) | ninf : v.w};
  }
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f16lo(unsigned d) {
  return (float)__builtin_bit_cast(f16x2, d).x;
}
__device__ __forceinline__ float f16hi(unsigned d) {
  return (float)__builtin_bit_cast(f16x2, d).y;
}
// float32 -> two float16, each rounded to nearest even (fp16 subnormals
// kept), packed low then high
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}

// IEEE binary16: widening to float32 is exact; narrowing rounds to nearest
// even.
template <>
struct Elem<_Float16> {
  static constexpr int VE = 8;
  static constexpr unsigned kNegInfWord = 0xFC00FC00u;
  __device__ static __forceinline__ void unpack(u32x4 v, float (&f)[8]) {
    f[0] = f16lo(v.x); f[1] = f16hi(v.x);
    f[2] = f16lo(v.y); f[3] = f16hi(v.y);
    f[4] = f16lo(v.z); f[5] = f16hi(v.z);
    f[6] = f16lo(v.w); f[7] = f16hi(v.w);
  }
  __device__ static __forceinline__ u32x4 pack(const float (&g)[8]) {
    return u32x4{pack_f16x2(g[0], g[1]), pack_f16x2(g[2], g[3]), pack_f16x2(g[4], g[5]),
                 pack_f16x2(g[6], g[7])};
  }
  __device__ static __forceinline__ float load1(const _Float16* p) {
    const unsigned short h = *reinterpret_cast<const unsigned short*>(p);
    return f16lo((unsigned)h);
  }
  __device__ static __forceinline__ void store1(_Float16* p, float g) {
    const unsigned d = pack_f16x2(g, 0.f);
    __builtin_nontemporal_store((unsigned short)(d & 0xffffu),
                                reinterpret_cast<unsigned short*>(p));
  }
  // the vector with element j (0..7) replaced by -inf (fp16 0xFC00)
  __device__ static __forceinline__ u32x4 kill(u32x4 v, int j) {
    const int d = j >> 1;
    const unsigned keep = (j & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    const unsigned ninf = (j & 1) ? 0xFC000000u : 0x0000FC00u;
    return u32x4{d == 0 ? (v.x & keep) | ninf : v.x, d == 1 ? (v.y & keep) | ninf : v.y,
                 d == 2 ? (v.z & keep) | ninf : v.z, d == 3 ? (v.w & keep) | ninf : v.w};
  }
};

// Element `half` of a 32-bit word, widened: float32 is the word itself;
// 16-bit types hold element 0 in the low half.  pack_word is the inverse
// (each element rounded to nearest even).
template <typename T>
__device__ __forceinline__ float widen_half(unsigned d, int half);
template <>
__device__ __forceinline__ float widen_half<float>(unsigned d, int) {
  return __builtin_bit_cast(float, d);
}
template <>
__device__ __forceinline__ float widen_half<__bf16>(unsigned d, int half) {
  return half ? bf16hi(d) : bf16lo(d);
}
template <>
__device__ __forceinline__ float widen_half<_Float16>(unsigned d, int half) {
  return half ? f16hi(d) : f16lo(d);
}
template <typename T>
__device__ __forceinline__ unsigned pack_word(const float* g);
template <>
__device__ __forceinline__ unsigned pack_word<float>(const float* g) {
  return __builtin_bit_cast(unsigned, g[0]);
}
template <>
__device__ __forceinline__ unsigned pack_word<__bf16>(const float* g) {
  return pack_bf16x2(g[0], g[1]);
}
template <>
__device__ __forceinline__ unsigned pack_word<_Float16>(const float* g) {
  return pack_f16x2(g[0], g[1]);
}

// ---------------------------------------------------------------------------
// Maximum of 16-bit floating-point values (bf16 or fp16) on their bit
// patterns, two per instruction (v_pk_max_i16 / v_pk_min_i16), with no
// widening.  Both formats are sign and magnitude, so compared as signed
// 16-bit integers:
//  - non-negative values order as their numbers do, and every negative
//    value (sign bit set) lies below every non-negative one: when a set
//    holds a value >= +0, its integer maximum is its numeric maximum;
//  - negative values order in reverse: when every value of a set is
//    negative, its numeric maximum is its integer minimum.
// The -inf pattern (bf16 0xFF80, fp16 0xFC00) lies above every finite
// negative pattern as an integer, so it is never the minimum of a set that
// holds a finite negative value.
// ---------------------------------------------------------------------------
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ s16x2 pk_max16(u32x4 w) {
  const s16x8 h = __builtin_bit_cast(s16x8, w);
  return __builtin_elementwise_max(__builtin_elementwise_max(h.s01, h.s23),
                                   __builtin_elementwise_max(h.s45, h.s67));
}
__device__ __forceinline__ s16x2 pk_min16(u32x4 w) {
  const s16x8 h = __builtin_bit_cast(s16x8, w);
  return __builtin_elementwise_min(__builtin_elementwise_min(h.s01, h.s23),
                                   __builtin_elementwise_min(h.s45, h.s67));
}

// ---------------------------------------------------------------------------
// Cross-lane reductions.  DPP moves inside rows of 16 lanes (quad
// permutations, half-row and row mirrors) are plain VALU operands; the step
// across the two 16-lane halves of a 32-lane group uses ds_swizzle, and the
// last step across the two 32-lane halves reads lanes 0 and 32.  Every lane
// ends with the same value, and the order of the operations is fixed, so a
// reduction is bitwise reproducible.  All lanes of the wave must be active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kSwizzleXor16 = 0x401F; // bitmask mode: lane ^ 16 within 32

struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const {
    return fmax2(a, b);
  }
};
struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// All-reduce over aligned segments of S lanes (S = 1, 2, 4, 8, 16 or 32;
// the last step swaps the halves of each 32 lanes through ds_swizzle).
template <int S, typename Op>
__device__ __forceinline__ float seg_allreduce(float v, Op op) {
  static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "segment size");
  if constexpr (S >= 2) v = op(v, dpp<kDppXor1>(v));
  if constexpr (S >= 4) v = op(v, dpp<kDppXor2>(v));
  if constexpr (S >= 8) v = op(v, dpp<kDppHalfMirror>(v));
  if constexpr (S >= 16) v = op(v, dpp<kDppMirror>(v));
  if constexpr (S >= 32)
    v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                    kSwizzleXor16)));
  return v;
}

// All-reduce over the whole 64-lane wave; the result is wave-uniform.
template <typename Op>
__device__ __forceinline__ float wave_allreduce(float v, Op op) {
  v = seg_allreduce<16>(v, op);
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                  kSwizzleXor16)));
  const float lo = __builtin_bit_cast(float,
                                      __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float hi = __builtin_bit_cast(float,
                                      __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  return op(lo, hi);
}

__device__ __forceinline__ float wave_uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------------------
// Online max / sum-of-exponentials state in the log2 domain.
//
//   c : a running maximum of round(z * log2 e) over the elements seen
//   s : sum over those elements of 2^(z * log2 e - c)
//
// The exponent z*log2e - c is formed with one fma, so z*log2e is never
// rounded on its own; rounding c itself only scales every term of a row by
// the same power of two, which cancels in softmax = term / sum and is
// removed from the loss by working with c directly.  When c grows, s is
// rescaled by 2^(c_old - c_new).
// ---------------------------------------------------------------------------
// Pairwise sum of N values in a fixed order: element i is added to element
// i + ceil(W/2) while W > 1 (an odd middle element waits one level).
template <int W, int N>
__device__ __forceinline__ void tree_level(float (&t)[N]) {
  if constexpr (W > 1) {
    constexpr int H = (W + 1) / 2;
#pragma unroll
    for (int i = 0; i < W / 2; ++i) t[i] = t[i] + t[i + H];
    tree_level<H, N>(t);
  }
}

template <int N>
__device__ __forceinline__ float tree_sum(const float (&a)[N]) {
  float t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = a[i];
  tree_level<N, N>(t);
  return t[0];
}

template <int N>
__device__ __forceinline__ float max_of(const float (&a)[N]) {
  float m = a[0];
  if constexpr (N == 1) return m;
  int i = 1;
#pragma unroll
  for (; i + 1 < N; i += 2) m = fmax3(m, a[i], a[i + 1]);
  if (i < N) m = fmax2(m, a[i]);
  return m;
}

// Fold N new elements into (c, s).  vmax is their maximum (taken before any
// element was masked out of the sum); masked elements hold -inf.  e
// receives each element's term 2^(f log2e - c_new).
template <int N>
__device__ __forceinline__ void online_fold_e(float& c, float& s, float vmax, const float (&f)[N],
                                              float (&e)[N]) {
  const float cn = fmax2(c, vmax * kLog2e);
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = exp2_hw(__builtin_fmaf(f[i], kLog2e, -cn));
  s = s * exp2_hw(c - cn) + tree_sum(e);
  c = cn;
}

template <int N>
__device__ __forceinline__ void online_fold(float& c, float& s, float vmax, const float (&f)[N]) {
  float e[N];
  online_fold_e(c, s, vmax, f, e);
}

}  // namespace ce
