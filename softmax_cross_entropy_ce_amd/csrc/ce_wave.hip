// Host side of path 5: configuration choice and the launches of
// ce_wave_kernel (ce_wave.h).
#include "ce_wave_host.h"

#include "ce.h"
#include "ce_launch.h"
#include "ce_wave.h"

namespace ce_wave {

namespace {

template <typename T, int VB, int LB, bool GRAD, int OP>
int launch_cfg(const T* z, const int32_t* t, int64_t B, int C, const ce::RowArgs& rs, T* g,
               float* l, hipStream_t st) {
  constexpr int R = LB >= 128 ? 1 : 128 / LB;
  constexpr int64_t rows_per_block = (ce::kWaveThreads / 64) * R;
  const int64_t blocks = (B + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  ce_host::launch((ce::ce_wave_kernel<T, VB, LB, GRAD, OP>), dim3((unsigned)blocks),
                     dim3(ce::kWaveThreads), 0, st, z, t, B, C, rs, g, l);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_LAUNCH;
}

template <typename T, int VB, bool GRAD, int OP>
int launch_lb(int lb, const T* z, const int32_t* t, int64_t B, int C, const ce::RowArgs& rs,
              T* g, float* l, hipStream_t st) {
  switch (lb) {
    case 16: return launch_cfg<T, VB, 16, GRAD, OP>(z, t, B, C, rs, g, l, st);
    case 32: return launch_cfg<T, VB, 32, GRAD, OP>(z, t, B, C, rs, g, l, st);
    case 64: return launch_cfg<T, VB, 64, GRAD, OP>(z, t, B, C, rs, g, l, st);
    case 128: return launch_cfg<T, VB, 128, GRAD, OP>(z, t, B, C, rs, g, l, st);
    case 256:
      if constexpr (VB >= 8) return launch_cfg<T, VB, 256, GRAD, OP>(z, t, B, C, rs, g, l, st);
      return CE_ERR_PATH;
    default: return CE_ERR_PATH;
  }
}

template <typename T, bool GRAD, int OP>
int launch_t(int vb, int lb, const void* z, const int32_t* t, int64_t B, int C,
             const ce::RowArgs& rs, void* g, float* l, hipStream_t st) {
  const T* zz = static_cast<const T*>(z);
  T* gg = static_cast<T*>(g);
  switch (vb) {
    case 16: return launch_lb<T, 16, GRAD, OP>(lb, zz, t, B, C, rs, gg, l, st);
    case 8: return launch_lb<T, 8, GRAD, OP>(lb, zz, t, B, C, rs, gg, l, st);
    case 4: return launch_lb<T, 4, GRAD, OP>(lb, zz, t, B, C, rs, gg, l, st);
    default: return CE_ERR_PATH;
  }
}

template <typename T>
int launch_op(int op, bool grad, int vb, int lb, const void* z, const int32_t* t, int64_t B,
              int C, const ce::RowArgs& rs, void* g, float* l, hipStream_t st) {
  switch (op) {
    case ce::kOpCE:
      return grad ? launch_t<T, true, ce::kOpCE>(vb, lb, z, t, B, C, rs, g, l, st)
                  : launch_t<T, false, ce::kOpCE>(vb, lb, z, t, B, C, rs, g, l, st);
    case ce::kOpSoftmax:
      return grad ? launch_t<T, true, ce::kOpSoftmax>(vb, lb, z, t, B, C, rs, g, l, st)
                  : CE_ERR_PATH;
    case ce::kOpShard:
      return grad ? CE_ERR_PATH : launch_t<T, false, ce::kOpShard>(vb, lb, z, t, B, C, rs, g, l, st);
    default: return CE_ERR_PATH;
  }
}

template <typename T, int VB, int LB>
int launch_bwd_cfg(const void* y, const void* dy, int64_t B, int C, void* dx, hipStream_t st) {
  constexpr int R = LB >= 64 ? 1 : 64 / LB;
  constexpr int64_t rows_per_block = (ce::kWaveThreads / 64) * R;
  const int64_t blocks = (B + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffffLL) return CE_ERR_SHAPE;
  ce_host::launch((ce::sm_bwd_wave_kernel<T, VB, LB>), dim3((unsigned)blocks),
                     dim3(ce::kWaveThreads), 0, st, static_cast<const T*>(y),
                     static_cast<const T*>(dy), B, C, static_cast<T*>(dx));
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_LAUNCH;
}

template <typename T, int VB>
int launch_bwd_lb(int lb, const void* y, const void* dy, int64_t B, int C, void* dx,
                  hipStream_t st) {
  switch (lb) {
    case 16: return launch_bwd_cfg<T, VB, 16>(y, dy, B, C, dx, st);
    case 32: return launch_bwd_cfg<T, VB, 32>(y, dy, B, C, dx, st);
    case 64: return launch_bwd_cfg<T, VB, 64>(y, dy, B, C, dx, st);
    case 128: return launch_bwd_cfg<T, VB, 128>(y, dy, B, C, dx, st);
    default: return CE_ERR_PATH;
  }
}

template <typename T>
int launch_bwd_t(int vb, int lb, const void* y, const void* dy, int64_t B, int C, void* dx,
                 hipStream_t st) {
  switch (vb) {
    case 16: return launch_bwd_lb<T, 16>(lb, y, dy, B, C, dx, st);
    case 8: return launch_bwd_lb<T, 8>(lb, y, dy, B, C, dx, st);
    case 4: return launch_bwd_lb<T, 4>(lb, y, dy, B, C, dx, st);
    default: return CE_ERR_PATH;
  }
}

}  // namespace

int bwd_lane_bytes(int64_t C, int es, int vb) {
  const int lb = lane_bytes(C, es, vb);
  return lb <= 128 ? lb : 0;
}

int launch_bwd(int dtype, int vb, const void* y, const void* dy, int64_t B, int C, void* dx,
               hipStream_t st) {
  const int es = dtype == CE_F32 ? 4 : 2;
  const int lb = bwd_lane_bytes(C, es, vb);
  if (lb == 0) return CE_ERR_PATH;
  switch (dtype) {
    case CE_F32: return launch_bwd_t<float>(vb, lb, y, dy, B, C, dx, st);
    case CE_BF16: return launch_bwd_t<__bf16>(vb, lb, y, dy, B, C, dx, st);
    case CE_F16: return launch_bwd_t<_Float16>(vb, lb, y, dy, B, C, dx, st);
    default: return CE_ERR_DTYPE;
  }
}

int lane_bytes(int64_t C, int es, int vb) {
  if (vb != 4 && vb != 8 && vb != 16) return 0;
  const int64_t rb = C * es;
  for (int lb = 16; lb <= 256; lb *= 2) {
    if (lb < vb || (int64_t)64 * lb < rb) continue;
    if (vb == 4 && lb > 128) return 0;
    return lb;
  }
  return 0;
}

int launch(int dtype, int op, bool grad, int vb, const void* logits, const int32_t* targets,
           int64_t B, int C, const ce::RowArgs& rs, void* out, float* rows_out, hipStream_t st) {
  const int es = dtype == CE_F32 ? 4 : 2;
  const int lb = lane_bytes(C, es, vb);
  if (lb == 0) return CE_ERR_PATH;
  switch (dtype) {
    case CE_F32:
      return launch_op<float>(op, grad, vb, lb, logits, targets, B, C, rs, out, rows_out, st);
    case CE_BF16:
      return launch_op<__bf16>(op, grad, vb, lb, logits, targets, B, C, rs, out, rows_out, st);
    case CE_F16:
      return launch_op<_Float16>(op, grad, vb, lb, logits, targets, B, C, rs, out, rows_out, st);
    default: return CE_ERR_DTYPE;
  }
}

}  // namespace ce_wave
