// prepack.hip -- canonical codes/scales -> gfx950 GEMV/MFMA layout, and the
// diagnostic read-back of the prepacked codes.
//
// The onnxruntime pull request 33005 (Description) prepacks expert weights
// once from the initializers and keeps the scales transposed for the
// kernels; here the prepacked layout is the one described in
// qmoe_internal.h (MatLayout): k-tiles of four 16-B chunks per row, laid out
// so that one 1 KiB wave load is the MFMA B operand of 16 rows, and the
// scales of a row's k-tile adjacent.
#include "qmoe_internal.h"
#include "codec.hpp"

namespace qmoe {

// One thread per (expert, row, chunk slot): 16 canonical bytes in, four
// prepacked dwords out (zeros for the padding chunks of a partial k-tile).
__global__ __launch_bounds__(256) void prepack_codes_kernel(MatLayout L, int64_t total,
                                                            const uint8_t *__restrict__ src,
                                                            uint8_t *__restrict__ dst,
                                                            uint32_t *__restrict__ err) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t NCP = 4 * L.NKT;  // chunk slots per row
  const int64_t c = idx % NCP;
  const int64_t n = (idx / NCP) % L.N;
  const int64_t e = idx / NCP / L.N;
  uint32_t out[4] = {0, 0, 0, 0};
  int bad = 0;
  if (c < L.NC) {
    const int64_t row_bytes = L.K * L.bits / 8;
    const uint8_t *s = src + (e * L.N + n) * row_bytes + c * kChunkBytes;
    uint8_t in[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) in[i] = s[i];
    const int fmask = (1 << L.bits) - 1;
    const int wpd = 32 / L.bits;  // weights per dword
    for (int k = 0; k < L.kc; ++k) {
      const int bit = k * L.bits;
      const uint32_t u = (in[bit >> 3] >> (bit & 7)) & fmask;
      if (L.qtype == QMOE_QTYPE_TERNARY && u == 3) bad = 1;
      const int d = k / wpd, kk = k % wpd, j = kk >> 1, hi = kk & 1;
      out[d] |= u << (L.bits * j + 16 * hi);
    }
  }
  uint8_t *o = dst + e * L.stride;
#pragma unroll
  for (int d = 0; d < 4; ++d) *reinterpret_cast<uint32_t *>(o + L.code_word_offset(n, c, d)) = out[d];
  if (bad) atomicAdd(err, 1u);
}

// One workgroup per (row group, expert).  The source of a row group is one
// contiguous [64 rows][nblk] block of the canonical scales.  A thread takes
// one (k-tile, row) pair, in destination order [k-tile][row], and writes its
// bpk block entries side by side (coalesced stores, index math once per
// pair); the reads stay inside the small source block (cache-resident).
// Entries past the last block are zero.
__global__ __launch_bounds__(256) void prepack_scales_kernel(MatLayout L, const uint16_t *__restrict__ scales,
                                                             const uint16_t *__restrict__ biases,
                                                             uint8_t *__restrict__ dst) {
  const int rg = blockIdx.x, e = blockIdx.y;
  const int nblk = (int)L.nblk, bpk = L.bpk;  // bpk in {1, 2, 4}
  const int pairs = (int)L.NKT * kLanes;      // (k-tile, row) pairs of one row group
  const int64_t src0 = ((int64_t)e * L.N + (int64_t)rg * kRowsPerGroup) * nblk;
  const int64_t dst0 = (int64_t)rg * pairs * bpk;
  uint8_t *base = dst + (int64_t)e * L.stride + L.scales_off;
  for (int q = threadIdx.x; q < pairs; q += blockDim.x) {
    const int row = q & (kLanes - 1), kt = q / kLanes;
    const int b0 = kt * bpk;
    const int64_t src = src0 + (int64_t)row * nblk + b0;
    const int64_t d = dst0 + (int64_t)q * bpk;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      if (bi >= bpk) break;
      const bool real = b0 + bi < nblk;
      if (L.affine)
        reinterpret_cast<uint32_t *>(base)[d + bi] =
            real ? ((uint32_t)scales[src + bi] | ((uint32_t)biases[src + bi] << 16)) : 0u;
      else
        reinterpret_cast<uint16_t *>(base)[d + bi] = real ? scales[src + bi] : (uint16_t)0;
    }
  }
}

// Diagnostic read-back through the same register decoders the kernels use.
// Both activation flavours (bf16 and f16 magic) must agree; a disagreement
// writes -128, which no valid code takes.  One thread per (expert, row, chunk).
template <int BITS>
__global__ __launch_bounds__(256) void unpack_codes_kernel(MatLayout L, int64_t total,
                                                           const uint8_t *__restrict__ src,
                                                           int8_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t c = idx % L.NC;
  const int64_t n = (idx / L.NC) % L.N;
  const int64_t e = idx / L.NC / L.N;
  const uint8_t *m = src + e * L.stride;
  uint32_t dw[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dw[d] = *reinterpret_cast<const uint32_t *>(m + L.code_word_offset(n, c, d));
  const int zp = qtype_zero_point(L.qtype);
  using CB = Codec<BITS, false>;
  using CF = Codec<BITS, true>;
  int8_t *o = out + (e * L.N + n) * L.K + c * L.kc;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t pb[CB::kPairs], pf[CF::kPairs];
    CB::extract(dw[d], pb);
    CF::extract(dw[d], pf);
#pragma unroll
    for (int j = 0; j < CB::kPairs; ++j) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const float ub = bf16_to_f32((pb[j] >> (16 * hi)) & 0xFFFFu) - CB::base(j);
        const float uf = f16_to_f32((pf[j] >> (16 * hi)) & 0xFFFFu) - CF::base(j);
        const int q = (int)ub - zp;
        o[d * CB::kPeriod + 2 * j + hi] = (ub == uf) ? (int8_t)q : (int8_t)-128;
      }
    }
  }
}

static inline unsigned nblocks(int64_t total, int bs) { return (unsigned)((total + bs - 1) / bs); }

hipError_t launch_prepack_matrix(const MatLayout &L, int E, const uint8_t *codes,
                                 const uint16_t *scales, const uint16_t *biases, uint8_t *dst,
                                 uint32_t *err_word, hipStream_t s) {
  const int64_t tc = (int64_t)E * L.N * 4 * L.NKT;
  hipLaunchKernelGGL(prepack_codes_kernel, dim3(nblocks(tc, 256)), dim3(256), 0, s, L, tc, codes, dst,
                     err_word);
  hipLaunchKernelGGL(prepack_scales_kernel, dim3((unsigned)L.RG, (unsigned)E), dim3(256), 0, s, L, scales, biases,
                     dst);
  return hipGetLastError();
}

hipError_t launch_prepack_scales(const MatLayout &L, int E, const uint16_t *scales, const uint16_t *biases,
                                 uint8_t *dst, hipStream_t s) {
  hipLaunchKernelGGL(prepack_scales_kernel, dim3((unsigned)L.RG, (unsigned)E), dim3(256), 0, s, L, scales, biases,
                     dst);
  return hipGetLastError();
}

hipError_t launch_unpack_matrix(const MatLayout &L, int E, const uint8_t *src, int8_t *codes_out,
                                hipStream_t s) {
  const int64_t tc = (int64_t)E * L.N * L.NC;
  if (L.bits == 4)
    hipLaunchKernelGGL(unpack_codes_kernel<4>, dim3(nblocks(tc, 256)), dim3(256), 0, s, L, tc, src,
                       codes_out);
  else
    hipLaunchKernelGGL(unpack_codes_kernel<2>, dim3(nblocks(tc, 256)), dim3(256), 0, s, L, tc, src,
                       codes_out);
  return hipGetLastError();
}

}  // namespace qmoe
