// grouped.hip -- preparation passes of the grouped larger-M path (per-row
// and per-expert power-of-two scales) and the dispatch of the grouped MFMA
// kernel over its epilogues (grouped_impl.hpp, one translation unit each).
#include "grouped_impl.hpp"

namespace qmoe {

hipError_t launch_grouped_swiglu(const GroupedArgs &a, int grid, hipStream_t s);
hipError_t launch_grouped_f32(const GroupedArgs &a, int grid, hipStream_t s);
hipError_t launch_grouped_act(const GroupedArgs &a, int grid, hipStream_t s);

// ---------------------------------------------------------------- prep
// One wave per row: power of two that brings max |x| below 2^14, and
// optionally the row times it as f16 (K is a multiple of 64, rows 16-B aligned).
__global__ __launch_bounds__(256) void rowscale_kernel(const uint16_t *__restrict__ x, int rows, int64_t K,
                                                       int in_f16, float *__restrict__ rowsc,
                                                       uint16_t *__restrict__ xs) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const uint4 *xr = reinterpret_cast<const uint4 *>(x + (int64_t)r * K);
  const int64_t n8 = K / 8;
  float m = 0.f;
  for (int64_t i = lane; i < n8; i += 64) {
    const uint4 v = xr[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) m = fmaxf(m, fabsf(half_to_f32_rt((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu, in_f16)));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float sc = pow2_below(m, 14);
  if (lane == 0) rowsc[r] = sc;
  if (xs == nullptr) return;
  uint4 *xo = reinterpret_cast<uint4 *>(xs + (int64_t)r * K);
  for (int64_t i = lane; i < n8; i += 64) {
    const uint4 v = xr[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    half8_t hv;
#pragma unroll
    for (int h = 0; h < 8; ++h) hv[h] = (_Float16)(half_to_f32_rt((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu, in_f16) * sc);
    xo[i] = __builtin_bit_cast(uint4, hv);
  }
}

// One wave per fp32 row: the bits of max |x| (non-negative floats order like
// their bits), which the grouped kernel turns into the row's power of two
// when it stages the row as f16 hi + lo parts.
__global__ __launch_bounds__(256) void rowmax_f32_kernel(const float *__restrict__ x, int rows, int64_t K,
                                                         uint32_t *__restrict__ rowmax) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const float4 *xr = reinterpret_cast<const float4 *>(x + (int64_t)r * K);
  float m = 0.f;
  for (int64_t i = lane; i < K / 4; i += 64) {
    const float4 v = xr[i];
    m = fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) rowmax[r] = __float_as_uint(m);
}

// One 1024-thread workgroup per expert: power of two that keeps
// max |s| * qmax below 2^15.  The prepacked scale section is read in 16-byte
// vectors (it is 256-B aligned and a multiple of 128 B long; padding
// entries are zero); affine entries hold the scale in their low half.
__global__ __launch_bounds__(1024) void wscale_kernel(MatLayout L, const uint8_t *__restrict__ mat,
                                                      float *__restrict__ wsc) {
  __shared__ float red[1024 / 64];
  const int e = blockIdx.x;
  const uint4 *sb = reinterpret_cast<const uint4 *>(mat + (int64_t)e * L.stride + L.scales_off);
  const int64_t nv = L.RG * L.NKT * kLanes * L.bpk * (L.affine ? 4 : 2) / 16;
  const int f16 = L.sdtype == QMOE_DTYPE_F16;
  float m = 0.f;
  for (int64_t i = threadIdx.x; i < nv; i += blockDim.x) {
    const uint4 v = sb[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m = fmaxf(m, fabsf(half_to_f32_rt(w[q] & 0xFFFFu, f16)));
      if (!L.affine) m = fmaxf(m, fabsf(half_to_f32_rt(w[q] >> 16, f16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) mm = fmaxf(mm, red[w]);
    wsc[e] = pow2_below(mm * (float)qtype_qmax(L.qtype), 15);
  }
}

// Few experts (the dense matrix is one) would leave most compute units idle
// with one workgroup each; there the same power of two comes from three
// stream-ordered passes over the same scale section: clear the per-expert
// maxima, take the maximum of |s| over slices of kWscaleSlice vectors of
// 16 B with one atomic per workgroup (|s| bits order like the values; NaN
// entries are skipped), then turn each maximum into the power of two in
// place.
constexpr int kWscaleSlice = 4096;       // 16-B vectors per workgroup (64 KiB)
constexpr int kWscalePerExpertMin = 32;  // from this many experts on: one workgroup per expert

__global__ __launch_bounds__(256) void wscale_clear_kernel(uint32_t *__restrict__ m, int E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) m[e] = 0u;
}

__global__ __launch_bounds__(256) void wscale_max_kernel(MatLayout L, const uint8_t *__restrict__ mat,
                                                         uint32_t *__restrict__ mbits) {
  __shared__ float red[256 / 64];
  const int e = blockIdx.y;
  const uint4 *sb = reinterpret_cast<const uint4 *>(mat + (int64_t)e * L.stride + L.scales_off);
  const int64_t nv = L.RG * L.NKT * kLanes * L.bpk * (L.affine ? 4 : 2) / 16;
  const int64_t v0 = (int64_t)blockIdx.x * kWscaleSlice;
  const int64_t v1 = v0 + kWscaleSlice < nv ? v0 + kWscaleSlice : nv;
  const int f16 = L.sdtype == QMOE_DTYPE_F16;
  float m = 0.f;
  for (int64_t i = v0 + threadIdx.x; i < v1; i += blockDim.x) {
    const uint4 v = sb[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m = fmaxf(m, fabsf(half_to_f32_rt(w[q] & 0xFFFFu, f16)));
      if (!L.affine) m = fmaxf(m, fabsf(half_to_f32_rt(w[q] >> 16, f16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float mm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(&mbits[e], __float_as_uint(mm));
  }
}

__global__ __launch_bounds__(256) void wscale_final_kernel(MatLayout L, float *__restrict__ wsc, int E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) wsc[e] = pow2_below(wsc[e] * (float)qtype_qmax(L.qtype), 15);  // wsc[e] holds max |s|
}

hipError_t launch_grouped(const GroupedArgs &a, int epilogue, int grid_tiles, hipStream_t s) {
  // the kernel's tile width (FC2 with its fp32 per-slot output has a shape of its own)
  const GroupedShape sh = grouped_shape(qtype_affine(a.qtype), a.tile_rows, epilogue == kGEpiStoreF32);
  const int tw = sh.nw * 16 * sh.nj;
  const int ntn = (int)((a.N + tw - 1) / tw);
  const int grid = grid_tiles * ntn;
  if (grid == 0) return hipSuccess;
  if (epilogue == kGEpiSwiGLU) return launch_grouped_swiglu(a, grid, s);
  if (epilogue == kGEpiStoreF32) return launch_grouped_f32(a, grid, s);
  return launch_grouped_act(a, grid, s);
}

hipError_t launch_rowscale(const void *x, int rows, int64_t K, int in_f16, float *rowsc, uint16_t *xs,
                           hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return qlaunch(rowscale_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, (const uint16_t *)x, rows, K, in_f16,
                 rowsc, xs);
}

// FC2's input, once for all column tiles: each fp32 row of h times its power
// of two (from the row's |max| bits, below 2^14) as f16 hi = RNE(h 2^r) and
// lo = RNE(h 2^r - hi), the same parts the grouped kernel would form while
// staging.  Written in place: each group of 8 k becomes [hi 8][lo 8] in the
// same 32 bytes, so one thread reads its group before writing it.
__global__ __launch_bounds__(256) void split_rows_kernel(float *__restrict__ h, int64_t groups, int64_t gpr,
                                                         const uint32_t *__restrict__ rowmax) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= groups) return;
  const float sc = pow2_below(__uint_as_float(rowmax[i / gpr]), 14);
  uint4 *g = reinterpret_cast<uint4 *>(h) + 2 * i;
  const uint4 w0 = g[0], w1 = g[1];
  const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  half8_t hi, lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xs = __uint_as_float(w[e]) * sc;
    hi[e] = (_Float16)xs;
    lo[e] = (_Float16)(xs - (float)hi[e]);
  }
  g[0] = __builtin_bit_cast(uint4, hi);
  g[1] = __builtin_bit_cast(uint4, lo);
}

hipError_t launch_split_rows(float *h, int rows, int64_t K, const uint32_t *rowmax, hipStream_t s) {
  const int64_t groups = (int64_t)rows * (K / 8);
  if (groups <= 0) return hipSuccess;
  return qlaunch(split_rows_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, h, groups, K / 8, rowmax);
}

hipError_t launch_rowmax_f32(const float *x, int rows, int64_t K, uint32_t *rowmax, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return qlaunch(rowmax_f32_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, rowmax);
}

hipError_t launch_wscale(const MatLayout &L, int E, const uint8_t *mat, float *wsc, hipStream_t s) {
  if (E >= kWscalePerExpertMin) return qlaunch(wscale_kernel, dim3(E), dim3(1024), 0, s, L, mat, wsc);
  // wsc holds the maxima' bits between the passes
  uint32_t *mbits = reinterpret_cast<uint32_t *>(wsc);
  const int64_t nv = L.RG * L.NKT * kLanes * L.bpk * (L.affine ? 4 : 2) / 16;
  const unsigned slices = (unsigned)((nv + kWscaleSlice - 1) / kWscaleSlice);
  hipError_t e = qlaunch(wscale_clear_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, mbits, E);
  if (e == hipSuccess && slices > 0)
    e = qlaunch(wscale_max_kernel, dim3(slices, (unsigned)E), dim3(256), 0, s, L, mat, mbits);
  if (e == hipSuccess) e = qlaunch(wscale_final_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, L, wsc, E);
  return e;
}

}  // namespace qmoe
