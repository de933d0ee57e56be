// gemv_impl.hpp -- register-accumulator quantized GEMV for M <= 16 rows.
//
// Computes out[m][n] = sum_k W[n][k] * in[m][k] for the rows m routed to one
// expert (or M dense rows), dequantizing every weight chunk once in VGPRs and
// applying it to all M rows held in per-lane accumulators.  This is the
// register-level answer to the per-token GEMV problem described on the
// inference-research gotcha page ("The QMoE sub-1-bit expert kernel is a
// GEMV ...": loop over the tokens inside the kernel instead of one GEMV per
// token) and the fused gate/up SwiGLU expert GEMV + separate down GEMV of
// onnx-genai pull request 1167.
//
// gfx950 mapping (not the pages' one-warp-per-row design):
//   - one output row per lane, 64 rows per wavefront: the prepacked layout
//     makes each chunk load a 1 KiB contiguous 16-B-per-lane read;
//   - the activations are identical across the lanes of a wave, so they are
//     read with scalar loads into SGPRs and used directly as the second
//     operand of v_dot2_f32_{bf16,f16} (no LDS traffic for x);
//   - the K dimension is split over the KS wavefronts of a workgroup; the
//     partial sums meet in LDS and are added in a fixed wavefront order;
//   - per block: D = sum (base + u) x by dot2, then acc += s * (D - C) (+ b X)
//     with C = sum (base + zero point) x and X = sum x computed once per row
//     and block in the workgroup prologue.
#pragma once

#include "codec.hpp"
#include "qmoe_internal.h"

namespace qmoe {

template <int QT>
struct QtTraits {
  static constexpr int kBits = (QT == QMOE_QTYPE_SYM_INT4 || QT == QMOE_QTYPE_AFFINE_INT4) ? 4 : 2;
  static constexpr bool kAffine = (QT == QMOE_QTYPE_AFFINE_INT2 || QT == QMOE_QTYPE_AFFINE_INT4);
  static constexpr int kZeroPoint = (QT == QMOE_QTYPE_SYM_INT4)   ? 8
                                    : (QT == QMOE_QTYPE_SYM_INT2) ? 2
                                    : (QT == QMOE_QTYPE_TERNARY)  ? 1
                                                                  : 0;
};

template <int QT, bool F16, int EPI, int MMAX, int BLOCK>
__global__ __launch_bounds__(512) void gemv_kernel(const GemvArgs a) {
  using TR = QtTraits<QT>;
  using CD = Codec<TR::kBits, F16>;
  constexpr int PPD = CD::kPairs;           // pairs per dword
  constexpr int PPC = 4 * PPD;              // pairs per 16-B chunk
  constexpr int KC = 2 * PPC;               // weights per chunk
  constexpr int CPB = BLOCK / KC;           // chunks per block
  static_assert(CPB >= 1, "block smaller than a chunk");
  constexpr int PB = (8 / CPB) > 0 ? (8 / CPB) : 1;  // blocks of loads in flight per wave
  constexpr int PARTS = (EPI == kEpiStoreF32) ? 2 : 1;  // FC2 reads h as bf16 hi + lo
  constexpr int EPT = BLOCK / 16;           // prologue: elements per thread per block

  extern __shared__ float smem[];
  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = threadIdx.x / kLanes;
  const int KS = blockDim.x / kLanes;
  const int slot = (int)(blockIdx.x / a.RG);
  const int64_t rg = blockIdx.x % a.RG;

  int e, M, pbase;
  if (a.dense_M > 0) {
    e = 0;
    M = a.dense_M;
    pbase = 0;
  } else {
    if (slot >= a.num_active[0]) return;
    e = a.active[slot];
    M = a.counts[e];
    pbase = a.offsets[e];
  }
  if (M > MMAX) M = MMAX;  // the host sizes MMAX >= every row count; clamp keeps accesses in bounds
  const int nblk = (int)a.nblk;
  float *s_corr = smem;                        // [MMAX][nblk][2]: C, X
  float *s_red = smem + MMAX * nblk * 2;       // [KS][MMAX][64]

  auto in_row = [&](int m) -> int64_t {
    if (a.dense_M > 0) return m;
    const int p = pbase + m;
    return a.in_gather_token ? (int64_t)(a.row_list[p] / a.top_k) : (int64_t)p;
  };

  // ---- prologue: C = sum (base_k + zp) x_k and X = sum x_k per row and block
  {
    const int nsum = M * nblk * 16;
    for (int idx = threadIdx.x; idx < nsum; idx += blockDim.x) {
      const int sub = idx & 15, pm = idx >> 4;
      const int m = pm / nblk, blk = pm % nblk;
      const int64_t k0 = (int64_t)blk * BLOCK + sub * EPT;
      float cs = 0.f, xs = 0.f;
#pragma unroll
      for (int part = 0; part < PARTS; ++part) {
        const uint16_t *xr = reinterpret_cast<const uint16_t *>(a.in + in_row(m) * a.in_row_pairs +
                                                                part * a.in_part_stride);
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          const int64_t k = k0 + i;
          const float xv = half_to_f32<F16>(xr[k]);
          const int j = (int)(k % CD::kPeriod) >> 1;
          cs = fmaf(CD::base(j) + (float)TR::kZeroPoint, xv, cs);
          xs += xv;
        }
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        cs += __shfl_xor(cs, off);
        xs += __shfl_xor(xs, off);
      }
      if (sub == 0) {
        s_corr[(m * nblk + blk) * 2 + 0] = cs;
        s_corr[(m * nblk + blk) * 2 + 1] = xs;
      }
    }
  }
  __syncthreads();

  // ---- main loop over this wave's blocks
  const int b0 = (int)((int64_t)wave * nblk / KS);
  const int b1 = (int)((int64_t)(wave + 1) * nblk / KS);
  const uint8_t *wexp = a.w + (int64_t)e * a.expert_stride;
  const uint4 *cptr = reinterpret_cast<const uint4 *>(wexp) + rg * a.NC * kLanes + lane;
  const uint8_t *sbase = wexp + a.scales_off;
  const int64_t sidx0 = rg * a.nblk * kLanes + lane;
  auto load_scale = [&](int b) -> uint32_t {
    if constexpr (TR::kAffine)
      return reinterpret_cast<const uint32_t *>(sbase)[sidx0 + (int64_t)b * kLanes];
    else
      return reinterpret_cast<const uint16_t *>(sbase)[sidx0 + (int64_t)b * kLanes];
  };

  const uint32_t *xrow[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) xrow[m] = a.in + (m < M ? in_row(m) : 0) * a.in_row_pairs;

  float acc[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) acc[m] = 0.f;

  uint4 cb[PB][CPB];
  uint32_t sb[PB];
#pragma unroll
  for (int i = 0; i < PB; ++i) {
    const int b = b0 + i;
    if (b < b1) {
#pragma unroll
      for (int ci = 0; ci < CPB; ++ci) cb[i][ci] = cptr[((int64_t)b * CPB + ci) * kLanes];
      sb[i] = load_scale(b);
    }
  }
  const bool sf16 = a.sdtype == QMOE_DTYPE_F16;
  for (int bb = b0; bb < b1; bb += PB) {
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int b = bb + i;
      if (b < b1) {
        uint4 wv[CPB];
#pragma unroll
        for (int ci = 0; ci < CPB; ++ci) wv[ci] = cb[i][ci];
        const uint32_t sv = sb[i];
        if (b + PB < b1) {
#pragma unroll
          for (int ci = 0; ci < CPB; ++ci) cb[i][ci] = cptr[((int64_t)(b + PB) * CPB + ci) * kLanes];
          sb[i] = load_scale(b + PB);
        }
        float D[MMAX];
#pragma unroll
        for (int m = 0; m < MMAX; ++m) D[m] = 0.f;
#pragma unroll
        for (int ci = 0; ci < CPB; ++ci) {
          uint32_t pr[4][PPD];
          CD::extract(wv[ci].x, pr[0]);
          CD::extract(wv[ci].y, pr[1]);
          CD::extract(wv[ci].z, pr[2]);
          CD::extract(wv[ci].w, pr[3]);
          const int64_t kp0 = ((int64_t)b * CPB + ci) * PPC;
#pragma unroll
          for (int m = 0; m < MMAX; ++m) {
            if (m < M) {
              float d = D[m];
#pragma unroll
              for (int part = 0; part < PARTS; ++part) {
                const uint32_t *xp = xrow[m] + kp0 + part * a.in_part_stride;
#pragma unroll
                for (int dd = 0; dd < 4; ++dd)
#pragma unroll
                  for (int j = 0; j < PPD; ++j) d = dot2<F16>(pr[dd][j], xp[dd * PPD + j], d);
              }
              D[m] = d;
            }
          }
        }
        const float s = half_to_f32_rt(sv & 0xFFFFu, sf16);
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
          if (m < M) {
            const float2 cx = reinterpret_cast<const float2 *>(s_corr)[m * nblk + b];
            acc[m] = fmaf(s, D[m] - cx.x, acc[m]);
            if constexpr (TR::kAffine) acc[m] = fmaf(half_to_f32_rt(sv >> 16, sf16), cx.y, acc[m]);
          }
        }
      }
    }
  }

  // ---- cross-wave reduction in a fixed order, then the epilogue
#pragma unroll
  for (int m = 0; m < MMAX; ++m)
    if (m < M) s_red[(wave * MMAX + m) * kLanes + lane] = acc[m];
  __syncthreads();
  for (int t = threadIdx.x; t < M * kLanes; t += blockDim.x) {
    const int m = t / kLanes, l = t & (kLanes - 1);
    float v = 0.f;
    for (int w = 0; w < KS; ++w) v += s_red[(w * MMAX + m) * kLanes + l];
    const int64_t n = rg * kRowsPerGroup + l;
    if constexpr (EPI == kEpiStoreF32) {
      a.out_f32[(int64_t)(pbase + m) * a.N + n] = v;
    } else if constexpr (EPI == kEpiStoreAct) {
      a.out_act[(int64_t)m * a.N + n] = f32_to_act(v, a.act_dtype == QMOE_DTYPE_F16);
    } else {
      // rows 2i (gate) and 2i+1 (up) sit in neighbouring lanes
      const float up = __shfl_xor(v, 1);
      if ((l & 1) == 0) {
        const float g = v;
        const float h = g / (1.f + expf(-g)) * up;
        const int64_t Ih = a.N / 2;
        const int64_t i = rg * (kRowsPerGroup / 2) + (l >> 1);
        const int64_t p = pbase + m;
        const uint16_t hi = f32_to_bf16_rne(h);
        a.h_hi[p * Ih + i] = hi;
        a.h_lo[p * Ih + i] = f32_to_bf16_rne(h - bf16_to_f32(hi));
        if (a.h_dbg) a.h_dbg[(int64_t)a.row_list[p] * Ih + i] = h;
      }
    }
  }
}

template <int QT, bool F16, int EPI, int MMAX>
hipError_t launch_gemv_block(const GemvArgs &a, int block, int waves, int grid_slots,
                             hipStream_t s) {
  const dim3 grid((unsigned)(grid_slots * a.RG));
  const dim3 thr((unsigned)(waves * kLanes));
  const size_t lds = gemv_lds_bytes(MMAX, a.nblk, waves);
  if (block == 64)
    hipLaunchKernelGGL((gemv_kernel<QT, F16, EPI, MMAX, 64>), grid, thr, lds, s, a);
  else
    hipLaunchKernelGGL((gemv_kernel<QT, F16, EPI, MMAX, 128>), grid, thr, lds, s, a);
  return hipGetLastError();
}

template <int QT, bool F16, int EPI>
hipError_t launch_gemv_m(const GemvArgs &a, int block, int mmax, int waves, int grid_slots,
                         hipStream_t s) {
  switch (mmax) {
    case 1: return launch_gemv_block<QT, F16, EPI, 1>(a, block, waves, grid_slots, s);
    case 2: return launch_gemv_block<QT, F16, EPI, 2>(a, block, waves, grid_slots, s);
    case 4: return launch_gemv_block<QT, F16, EPI, 4>(a, block, waves, grid_slots, s);
    case 8: return launch_gemv_block<QT, F16, EPI, 8>(a, block, waves, grid_slots, s);
    default: return launch_gemv_block<QT, F16, EPI, 16>(a, block, waves, grid_slots, s);
  }
}

template <int QT>
hipError_t launch_gemv_qt(const GemvArgs &a, int epilogue, int in_f16, int mmax, int waves,
                          int grid_slots, hipStream_t s) {
  const int block = (int)(a.K / a.nblk);
  if (epilogue == kEpiStoreF32)
    return launch_gemv_m<QT, false, kEpiStoreF32>(a, block, mmax, waves, grid_slots, s);
  if (epilogue == kEpiSwiGLU)
    return in_f16 ? launch_gemv_m<QT, true, kEpiSwiGLU>(a, block, mmax, waves, grid_slots, s)
                  : launch_gemv_m<QT, false, kEpiSwiGLU>(a, block, mmax, waves, grid_slots, s);
  return in_f16 ? launch_gemv_m<QT, true, kEpiStoreAct>(a, block, mmax, waves, grid_slots, s)
                : launch_gemv_m<QT, false, kEpiStoreAct>(a, block, mmax, waves, grid_slots, s);
}

}  // namespace qmoe
