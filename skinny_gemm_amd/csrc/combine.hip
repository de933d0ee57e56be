// combine.hip -- top-k weighted combine back to token order (the finalize
// step of onnxruntime pull request 33005, Description), and the GEMV
// dispatch over quantization formats.
//
// y[t][n] = sum_{j=0..k-1} w[t][j] * o[pos(t, j)][n], summed in fp32 in
// ascending j from 0, rounded once to nearest-even in the activation dtype
// (stored as is for f32 activations).
// o holds the per-slot FC2 outputs in expert-sorted order; pos is the
// inverse of the row list.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "codec.hpp"
#include "qmoe_internal.h"

namespace qmoe {

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const float *__restrict__ w, int T, int k,
                                                      int H, int act_dtype, void *__restrict__ y) {
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
  if (act_dtype == QMOE_DTYPE_F32) {
    reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + (int64_t)t * H)[n4] = acc;
    return;
  }
  const int is_f16 = act_dtype == QMOE_DTYPE_F16;
  uint2 out;
  out.x = (uint32_t)f32_to_act(acc.x, is_f16) | ((uint32_t)f32_to_act(acc.y, is_f16) << 16);
  out.y = (uint32_t)f32_to_act(acc.z, is_f16) | ((uint32_t)f32_to_act(acc.w, is_f16) << 16);
  reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(y) + (int64_t)t * H)[n4] = out;
}

// f32 rows -> bf16 hi + lo rows (hi = x rounded to nearest-even, lo = the
// rest rounded the same way), the two-part A operand of the GEMV.
__global__ __launch_bounds__(256) void split_f32_kernel(const float *__restrict__ x, int64_t n,
                                                        uint16_t *__restrict__ hi, uint16_t *__restrict__ lo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  const uint16_t h = f32_to_bf16_rne(v);
  hi[i] = h;
  lo[i] = f32_to_bf16_rne(v - bf16_to_f32(h));
}

hipError_t launch_split_f32(const float *x, int64_t n, uint16_t *hi, uint16_t *lo, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return qlaunch(split_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, n, hi, lo);
}

hipError_t launch_combine(const float *o, const int32_t *slot_pos, const float *w, int T, int k,
                          int H, int act_dtype, void *y, hipStream_t s) {
  const int64_t total = (int64_t)T * (H / 4);
  if (total == 0) return hipSuccess;
  return qlaunch(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, o, slot_pos, w, T, k, H,
                 act_dtype, y);
}

// Streaming read of n16 16-byte vectors: each lane issues four independent
// 16-B loads per round (each wave instruction covers 1 KiB contiguous) over a
// grid-stride sweep.  The XOR of every word read is stored only if it equals
// `never`, which the caller picks so that it does not occur, so the loads
// stay and the kernel writes nothing: its time is the read time.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4 *__restrict__ src, int64_t n16,
                                                         uint32_t never, uint32_t *__restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == never) sink[0] = acc;
}

hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int cus, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((int64_t)cus * 8, (n16 + 255) / 256);
  return qlaunch(read_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint4 *)src, n16,
                 0x9E3779B9u, sink);
}

const void *gemv_ptr_sym_int4(int, int, int, int, int, int);
const void *gemv_ptr_sym_int2(int, int, int, int, int, int);
const void *gemv_ptr_ternary(int, int, int, int, int, int);
const void *gemv_ptr_affine_int2(int, int, int, int, int, int);
const void *gemv_ptr_affine_int4(int, int, int, int, int, int);

const void *gemv_kernel_ptr(int qtype, int epilogue, int in_f16, int rows, int block, int tn, int ext) {
  switch (qtype) {
    case QMOE_QTYPE_SYM_INT4: return gemv_ptr_sym_int4(epilogue, in_f16, rows, block, tn, ext);
    case QMOE_QTYPE_SYM_INT2: return gemv_ptr_sym_int2(epilogue, in_f16, rows, block, tn, ext);
    case QMOE_QTYPE_TERNARY: return gemv_ptr_ternary(epilogue, in_f16, rows, block, tn, ext);
    case QMOE_QTYPE_AFFINE_INT2: return gemv_ptr_affine_int2(epilogue, in_f16, rows, block, tn, ext);
    default: return gemv_ptr_affine_int4(epilogue, in_f16, rows, block, tn, ext);
  }
}

hipError_t launch_gemv(const GemvArgs &a, int epilogue, int in_f16, int rows, int waves, int tn, int block,
                       int grid_slots, hipStream_t s) {
  // the EXT instances (bias, ReLU, unnormalised routed weights) only when the call uses them
  const void *fn = gemv_kernel_ptr(a.qtype, epilogue, in_f16, rows, block, tn,
                                   a.bias != nullptr || a.relu != 0 || a.route_softmax_all != 0 ||
                                       a.sw_custom != 0);
  if (fn == nullptr) return hipErrorInvalidConfiguration;  // no kernel for this (rows, tn) pairing
  GemvArgs args = a;
  void *kargs[] = {&args};
  const size_t lds = gemv_lds_bytes(rows, epilogue, waves, tn) +
                     (epilogue == kEpiDownCat && a.cat_stage ? gemv_cat_stage_bytes(a.route_k, a.K) : 0);
  return launch_raw(fn, dim3((unsigned)(grid_slots * a.RG * (4 / tn))), dim3((unsigned)(waves * kLanes)), kargs,
                    lds, s);
}

int gemv_blocks_per_cu(int qtype, int epilogue, int in_f16, int rows, int waves, int tn, int block) {
  const void *fn = gemv_kernel_ptr(qtype, epilogue, in_f16, rows, block, tn, 0);
  if (fn == nullptr) return 0;
  const size_t lds = gemv_lds_bytes(rows, epilogue, waves, tn);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  // the runtime query is not free: remember it per (device, kernel, waves)
  static std::mutex mu;
  static std::map<std::tuple<int, const void *, int, size_t>, int> cache;
  const auto key = std::make_tuple(dev, fn, waves, lds);
  {
    std::lock_guard<std::mutex> g(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, waves * kLanes, lds) != hipSuccess) {
    (void)hipGetLastError();
    n = 0;
  }
  std::lock_guard<std::mutex> g(mu);
  cache[key] = n;
  return n;
}

}  // namespace qmoe
