// combine.hip -- top-k weighted combine back to token order (the finalize
// step of onnxruntime pull request 33005, Description), and the GEMV
// dispatch over quantization formats.
//
// y[t][n] = sum_{j=0..k-1} w[t][j] * o[pos(t, j)][n], summed in fp32 in
// ascending j from 0, rounded once to nearest-even in the activation dtype.
// o holds the per-slot FC2 outputs in expert-sorted order; pos is the
// inverse of the row list.
#include "codec.hpp"
#include "qmoe_internal.h"

namespace qmoe {

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const float *__restrict__ w, int T, int k,
                                                      int H, int is_f16, uint16_t *__restrict__ y) {
  const int H4 = H / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * H4) return;
  const int t = (int)(idx / H4), n4 = (int)(idx % H4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int64_t r = (int64_t)t * k + j;
    const float wt = w[r];
    const float4 v = reinterpret_cast<const float4 *>(o + (int64_t)slot_pos[r] * H)[n4];
    acc.x = fmaf(wt, v.x, acc.x);
    acc.y = fmaf(wt, v.y, acc.y);
    acc.z = fmaf(wt, v.z, acc.z);
    acc.w = fmaf(wt, v.w, acc.w);
  }
  uint2 out;
  out.x = (uint32_t)f32_to_act(acc.x, is_f16) | ((uint32_t)f32_to_act(acc.y, is_f16) << 16);
  out.y = (uint32_t)f32_to_act(acc.z, is_f16) | ((uint32_t)f32_to_act(acc.w, is_f16) << 16);
  reinterpret_cast<uint2 *>(y + (int64_t)t * H)[n4] = out;
}

hipError_t launch_combine(const float *o, const int32_t *slot_pos, const float *w, int T, int k,
                          int H, int act_dtype, uint16_t *y, hipStream_t s) {
  const int64_t total = (int64_t)T * (H / 4);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, o,
                     slot_pos, w, T, k, H, act_dtype == QMOE_DTYPE_F16 ? 1 : 0, y);
  return hipGetLastError();
}

hipError_t launch_gemv_sym_int4(const GemvArgs &, int, int, int, int, int, hipStream_t);
hipError_t launch_gemv_sym_int2(const GemvArgs &, int, int, int, int, int, hipStream_t);
hipError_t launch_gemv_ternary(const GemvArgs &, int, int, int, int, int, hipStream_t);
hipError_t launch_gemv_affine_int2(const GemvArgs &, int, int, int, int, int, hipStream_t);
hipError_t launch_gemv_affine_int4(const GemvArgs &, int, int, int, int, int, hipStream_t);

hipError_t launch_gemv(const GemvArgs &a, int epilogue, int in_f16, int mmax, int waves,
                       int grid_slots, hipStream_t s) {
  switch (a.qtype) {
    case QMOE_QTYPE_SYM_INT4: return launch_gemv_sym_int4(a, epilogue, in_f16, mmax, waves, grid_slots, s);
    case QMOE_QTYPE_SYM_INT2: return launch_gemv_sym_int2(a, epilogue, in_f16, mmax, waves, grid_slots, s);
    case QMOE_QTYPE_TERNARY: return launch_gemv_ternary(a, epilogue, in_f16, mmax, waves, grid_slots, s);
    case QMOE_QTYPE_AFFINE_INT2:
      return launch_gemv_affine_int2(a, epilogue, in_f16, mmax, waves, grid_slots, s);
    default: return launch_gemv_affine_int4(a, epilogue, in_f16, mmax, waves, grid_slots, s);
  }
}

}  // namespace qmoe
