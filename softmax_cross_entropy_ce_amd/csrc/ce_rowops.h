// Per-row arithmetic and operations shared by the gfx950 kernels of the fused
// softmax cross-entropy path.
//
// The method (rumus project page, milestone M7a; rumus 0.1.1
// cross_entropy.wgsl pass 1 steps 1-4 and pass 2): per row, the max and the
// sum of exponentials give the log-sum-exp, the per-row loss is
// (lse - z_t) / B and the gradient is (softmax - onehot) / B; the per-row
// losses are then summed.  The WGSL kernel reads each row three times with
// one 64-lane workgroup per row and two shared-memory trees; the kernels
// here read each row from HBM once and write each gradient element once.
//
// Per row they compute, in float32 and the log2 domain:
//   cg     = round(max_c z_c * log2 e)
//   Sx     = sum_{c != t} 2^(z_c log2e - cg)      (target left out of the sum)
//   a_t    = z_t log2e - cg,  E_t = 2^a_t,  S = Sx + E_t
//   g_c    = 2^(z_c log2e - cg) / (S B)           (c != t)
//   g_t    = -Sx / (S B)                           (= (softmax_t - 1)/B without cancellation)
//   loss*B = log1p(Sx / E_t)                       when a_t > -60
//          = ln2 * (log2 S - a_t)                  otherwise
// Both forms equal ln(S / E_t) = lse - z_t; the first keeps full relative
// accuracy when the target holds almost all of the mass.
#pragma once

#include "ce_device.h"

namespace ce {

// What a row kernel computes from a row's max and sum of exponentials.
//   kOpCE       the fused cross-entropy: per-row loss and gradient
//               (softmax - onehot) / B.
//   kOpSoftmax  the row-wise softmax (rumus project page, milestone M8c) and,
//               where loss_rows is not null, the row's log-sum-exp.  No
//               targets are read.
//   kOpShard    the record of one vocabulary shard per row (the columns
//               [col0, col0 + C) of a longer row): its max, its sum of
//               exponentials without the target and the target logit where
//               the shard holds it.  No per-element output.
enum RowOp : int { kOpCE = 0, kOpSoftmax = 1, kOpShard = 2 };

// Per-call arguments of the row kernels.
//   invB        1/B, the scale of the batch mean (unless kept is set).
//   gmul        the upstream gradient of the loss, a device scalar that
//               multiplies the gradient (null: 1).
//   col0        kOpShard: the shard's first column in the whole row.
//   ldz, ldg    row strides of the logits and of the output, in elements
//               (>= C; equal to C for contiguous rows).
//   kept        device count of the rows that are not ignored; when set,
//               the mean is over those rows: the scale is 1/kept.
//   ignore      with has_ignore, rows whose target equals it are ignored
//               (kOpCE): loss 0 and a zero gradient row.
struct RowArgs {
  float invB;
  const float* gmul;
  int64_t col0;
  int64_t ldz, ldg;
  const uint32_t* kept;
  int32_t ignore;
  int32_t has_ignore;
};

__device__ __forceinline__ float row_invB(const RowArgs& rs) {
  return rs.kept != nullptr ? 1.0f / (float)*rs.kept : rs.invB;
}

// The target of a row as one call sees it: its column in the row (-1 when
// the row has none here), whether the row has a result and whether it is
// ignored.  A CE row has a result when its target lies in [0, C) or is the
// ignored value; a shard row always has a record (whether the target is
// valid at all is decided when the records are combined).
struct RowTarget {
  int t;
  bool valid;
  bool ignored;
};

// The same from the row's target value itself (raw: targets[row], loaded by
// the caller; unused for the softmax).
template <int OP>
__device__ __forceinline__ RowTarget row_target_of(int32_t raw, int C, const RowArgs& rs) {
  if constexpr (OP == kOpSoftmax) {
    return RowTarget{-1, true, false};
  } else {
    if (OP == kOpCE && rs.has_ignore && raw == rs.ignore) return RowTarget{-1, true, true};
    const int64_t t = (int64_t)raw - (OP == kOpShard ? rs.col0 : 0);
    const bool in = t >= 0 && t < C;
    return RowTarget{in ? (int)t : -1, OP == kOpShard || in, false};
  }
}

template <int OP>
__device__ __forceinline__ RowTarget row_target(const int32_t* targets, int64_t row, int C,
                                                const RowArgs& rs) {
  if constexpr (OP == kOpSoftmax) {
    return RowTarget{-1, true, false};
  } else {
    return row_target_of<OP>(targets[row], C, rs);
  }
}

// A shard's per-row record, four floats (c, sx, zt, own): c = max z * log2(e)
// rounded to float32, sx = the sum over the shard's non-target columns of
// 2^(z log2e - c), zt = the target logit (0 where the shard does not hold
// the target), own = 1 where it does, else 0.

__device__ __forceinline__ float grad_mul(const RowArgs& rs) {
  return rs.gmul != nullptr ? *rs.gmul : 1.0f;
}

// Per-row epilogue shared by all kernels: from the row's (cg, Sx) and the
// target logit, the gradient scale gmul/(S B) and the target's gradient.
// The per-row value (the loss, or the softmax's log-sum-exp) is formed by
// row_value only in the thread that stores it: its log1p is a long
// instruction sequence that the other threads of a row need not run.
struct RowResult {
  float scale;   // multiply 2^(z log2e - cg) by this to get the gradient
  float scale0;  // the same without the upstream factor gmul: 1/(S B)
  float gt;      // gradient of the target element
  float at, sx, invB;  // inputs of the per-row value (softmax: at = cg)
  int state;     // 0: a result; 1: target out of range (NaN); 2: ignored (0)
};

__device__ __forceinline__ RowResult row_epilogue(float cg, float sx, float zt, bool valid,
                                                  float invB, float gmul) {
  RowResult r;
  r.at = __builtin_fmaf(zt, kLog2e, -cg);
  const float S = sx + exp2_hw(r.at);
  // one v_rcp_f32 (within an ulp) rather than a correctly rounded divide:
  // S >= 1 and the gradient's bar is far wider than an fp32 ulp
  const float scale0 = invB * __builtin_amdgcn_rcpf(S);
  const float qnan = __builtin_nanf("");
  r.scale0 = valid ? scale0 : qnan;
  r.scale = valid ? scale0 * gmul : qnan;
  r.gt = valid ? -sx * r.scale : qnan;
  r.sx = sx;
  r.invB = invB;
  r.state = valid ? 0 : 1;
  return r;
}

// The per-row loss of a CE row, already scaled by 1/B: ln(S / E_t), as
// log1p(Sx / E_t) while E_t is not tiny (full relative accuracy when the
// target holds almost all of the mass), else ln2 (log2 S - a_t).
__device__ __forceinline__ float row_loss(const RowResult& r) {
  if (r.state == 2) return 0.f;
  if (r.state == 1) return __builtin_nanf("");
  float lossB;
  if (r.at > -60.f)
    lossB = log1pf(r.sx * exp2_hw(-r.at));
  else
    lossB = kLn2 * (log2_hw(r.sx + exp2_hw(r.at)) - r.at);
  return lossB * r.invB;
}

// The epilogue of each operation.  CE: row_epilogue, and an ignored row
// gets scale, target gradient and loss 0.  Softmax: scale = 1 / S (the
// target fields are unused, S = sx) and the per-row value is the
// log-sum-exp ln2 * (cg + log2 S).  Shard records need no epilogue.
template <int OP>
__device__ __forceinline__ RowResult row_finish(float cg, float sx, float zt, bool valid,
                                                bool ignored, float invB, float gmul) {
  if constexpr (OP == kOpCE) {
    RowResult r = row_epilogue(cg, sx, zt, valid, invB, gmul);
    if (ignored) {
      r.scale = r.scale0 = r.gt = 0.f;
      r.state = 2;
    }
    return r;
  } else {
    RowResult r;
    r.scale = r.scale0 = OP == kOpSoftmax ? 1.0f / sx : 0.f;
    r.gt = 0.f;
    r.at = cg;
    r.sx = sx;
    r.invB = invB;
    r.state = 0;
    return r;
  }
}

// The per-row value of each operation, evaluated where it is stored: CE
// the loss, softmax the log-sum-exp.
template <int OP>
__device__ __forceinline__ float row_value(const RowResult& r) {
  if constexpr (OP == kOpCE) {
    return row_loss(r);
  } else {
    return kLn2 * (r.at + log2_hw(r.sx));
  }
}

// The per-row output of each operation: CE the loss, softmax the
// log-sum-exp (when out is not null), a shard its record (out holds
// ShardRecords).
template <int OP>
__device__ __forceinline__ void store_row(float* out, int64_t row, const RowResult& rr, float cg,
                                          float sx, float zt, bool has_t) {
  if constexpr (OP == kOpCE) {
    out[row] = row_value<OP>(rr);
  } else if constexpr (OP == kOpSoftmax) {
    if (out != nullptr) out[row] = row_value<OP>(rr);
  } else {
    const f32x4 rec = {cg, sx, has_t ? zt : 0.f, has_t ? 1.f : 0.f};
    *reinterpret_cast<f32x4*>(out + 4 * row) = rec;
  }
}

// ---------------------------------------------------------------------------
// Loads and stores of VW consecutive elements (VW * sizeof(T) bytes, a power
// of two up to 16) through a buffer resource, widened to float32 and
// rounded back to the storage type to nearest even.  Out-of-range offsets
// read zeros and drop their stores (the resource's size bounds them).
// ---------------------------------------------------------------------------
template <typename T, int VW>
struct VecIO;

template <int VW>
struct VecIO<float, VW> {
  static_assert(VW == 1 || VW == 2 || VW == 4, "fp32 vector width");
  __device__ static __forceinline__ void load(rsrc_t r, uint32_t off, float (&f)[VW]) {
    if constexpr (VW == 1) {
      const unsigned d = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicyStream);
      f[0] = __builtin_bit_cast(float, d);
    } else if constexpr (VW == 2) {
      const f32x2 v = as_f32(__builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyStream));
      f[0] = v.x;
      f[1] = v.y;
    } else {
      const f32x4 v = as_f32(__builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyStream));
      f[0] = v.x;
      f[1] = v.y;
      f[2] = v.z;
      f[3] = v.w;
    }
  }
  __device__ static __forceinline__ void store(rsrc_t r, uint32_t off, const float (&g)[VW]) {
    if constexpr (VW == 1) {
      const float x = g[0];
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, (int)off, 0,
                                            kPolicyStream);
    } else if constexpr (VW == 2) {
      __builtin_amdgcn_raw_buffer_store_b64(as_u32(f32x2{g[0], g[1]}), r, (int)off, 0,
                                            kPolicyStream);
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(as_u32(f32x4{g[0], g[1], g[2], g[3]}), r, (int)off,
                                             0, kPolicyStream);
      wide_store_guard();
    }
  }
};

template <int VW>
struct VecIO<_Float16, VW> {
  static_assert(VW == 1 || VW == 2 || VW == 4 || VW == 8, "fp16 vector width");
  __device__ static __forceinline__ void load(rsrc_t r, uint32_t off, float (&f)[VW]) {
    if constexpr (VW == 1) {
      unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, kPolicyStream);
      f[0] = f16lo((unsigned)h);
    } else if constexpr (VW == 2) {
      unsigned d = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicyStream);
      f[0] = f16lo(d);
      f[1] = f16hi(d);
    } else if constexpr (VW == 4) {
      u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyStream);
      f[0] = f16lo(v.x); f[1] = f16hi(v.x);
      f[2] = f16lo(v.y); f[3] = f16hi(v.y);
    } else {
      u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyStream);
      float t[8];
      Elem<_Float16>::unpack(v, t);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = t[i];
    }
  }
  __device__ static __forceinline__ void store(rsrc_t r, uint32_t off, const float (&g)[VW]) {
    if constexpr (VW == 1) {
      unsigned d = pack_f16x2(g[0], 0.f);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(d & 0xffffu), r, (int)off, 0,
                                            kPolicyStream);
    } else if constexpr (VW == 2) {
      __builtin_amdgcn_raw_buffer_store_b32(pack_f16x2(g[0], g[1]), r, (int)off, 0,
                                            kPolicyStream);
    } else if constexpr (VW == 4) {
      u32x2 v = {pack_f16x2(g[0], g[1]), pack_f16x2(g[2], g[3])};
      __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kPolicyStream);
    } else {
      u32x4 v = {pack_f16x2(g[0], g[1]), pack_f16x2(g[2], g[3]), pack_f16x2(g[4], g[5]),
                 pack_f16x2(g[6], g[7])};
      __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kPolicyStream);
      wide_store_guard();
    }
  }
};

template <int VW>
struct VecIO<__bf16, VW> {
  static_assert(VW == 1 || VW == 2 || VW == 4 || VW == 8, "bf16 vector width");
  __device__ static __forceinline__ void load(rsrc_t r, uint32_t off, float (&f)[VW]) {
    if constexpr (VW == 1) {
      unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, kPolicyStream);
      f[0] = __builtin_bit_cast(float, (unsigned)h << 16);
    } else if constexpr (VW == 2) {
      unsigned d = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicyStream);
      f[0] = bf16lo(d);
      f[1] = bf16hi(d);
    } else if constexpr (VW == 4) {
      u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyStream);
      f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
      f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
    } else {
      u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyStream);
      float t[8];
      Elem<__bf16>::unpack(v, t);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = t[i];
    }
  }
  __device__ static __forceinline__ void store(rsrc_t r, uint32_t off, const float (&g)[VW]) {
    if constexpr (VW == 1) {
      unsigned d = pack_bf16x2(g[0], 0.f);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(d & 0xffffu), r, (int)off, 0,
                                            kPolicyStream);
    } else if constexpr (VW == 2) {
      __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(g[0], g[1]), r, (int)off, 0,
                                            kPolicyStream);
    } else if constexpr (VW == 4) {
      u32x2 v = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
      __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kPolicyStream);
    } else {
      u32x4 v = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                 pack_bf16x2(g[6], g[7])};
      __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kPolicyStream);
      wide_store_guard();
    }
  }
};

}  // namespace ce
