// gemv_impl.hpp -- register-accumulator quantized GEMV for M <= 16 rows.
//
// Computes out[m][n] = sum_k W[n][k] * in[m][k] for the rows m routed to one
// expert (or M dense rows), dequantizing every weight chunk once in VGPRs and
// applying it to all M rows held in per-lane accumulators.  This is the
// register-level answer to the per-token GEMV problem of the inference-research
// gotcha page on QMoE ("The QMoE sub-1-bit expert kernel is a GEMV ...": loop
// over the tokens that share an expert inside the kernel instead of one GEMV
// per token) and the fused gate/up SwiGLU expert GEMV + down GEMV of
// onnx-genai pull request 1167.
//
// gfx950 mapping (the pages' designs use one warp per row; here):
//   - one output row per lane, 64 rows per wavefront: every chunk load of the
//     prepacked layout is a 1 KiB contiguous read of 16 B per lane;
//   - the activations are the same for all lanes of a wave: for up to 4 rows
//     the workgroup stages them in LDS while the weight loads are in flight
//     and every lane reads the same address (broadcast ds_read_b128); for more
//     rows they are read with scalar loads into SGPRs and used directly as the
//     second operand of v_dot2_f32_{bf16,f16};
//   - K is split over the KS wavefronts of a workgroup; each wave issues all
//     of its weight and scale loads (up to 8 x 16 B per lane) before any
//     use, and the partial sums meet in LDS, added in a fixed wave order;
//   - per block: D = sum (base + u) x by dot2, acc += s * (D - C) (+ b X), with
//     C = sum (base + zero point) x and X = sum x computed once per row and
//     block by the workgroup while the weight loads are in flight.
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
  constexpr int BPW = CPB >= 8 ? 1 : 8 / CPB;          // blocks per load batch (8 chunks)
  constexpr int PARTS = (EPI == kEpiDown) ? 2 : 1;  // FC2 reads h as bf16 hi + lo
  constexpr int EPT = BLOCK / 16;           // prologue: elements per thread per block
  constexpr bool XLDS = MMAX <= kGemvLdsRows;  // activations staged in LDS

  extern __shared__ float smem[];
  const int lane = threadIdx.x & (kLanes - 1);
  // wave index made provably uniform so activation addresses stay scalar (s_load)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int KS = blockDim.x / kLanes;
  const int RG = (int)a.RG;
  const int slot = (int)blockIdx.x / RG;
  const int rg = (int)blockIdx.x - slot * RG;

  int e, M, pbase;
  if (a.dense_M > 0) {
    e = 0;
    M = a.dense_M;
    pbase = 0;
  } else {
    const int4 si = a.slot_info[slot];
    e = si.x;
    M = si.y;
    pbase = si.z;
    if (M <= 0) return;
  }
  if (M > MMAX) M = MMAX;  // the host sizes MMAX >= every row count; the clamp keeps accesses in bounds
  const int nblk = (int)a.nblk;
  const int Kp = (int)(a.K / 2);               // pairs per row
  // LDS: staged activations first (16-B aligned for ds_read_b128), then the
  // block corrections and the cross-wave partial sums
  uint32_t *s_x = reinterpret_cast<uint32_t *>(smem);                 // [PARTS][MMAX][Kp]
  float *s_corr = smem + (XLDS ? PARTS * MMAX * Kp : 0);              // [MMAX][nblk][2]: C, X
  float *s_red = s_corr + MMAX * nblk * 2;                            // [KS][MMAX][64]

  // ---- 1. this wave's weight and scale loads, all issued before any use
  const int b0 = (int)((int64_t)wave * nblk / KS);
  const int b1 = (int)((int64_t)(wave + 1) * nblk / KS);
  const uint8_t *wexp = a.w + (int64_t)e * a.expert_stride;
  const uint4 *cptr = reinterpret_cast<const uint4 *>(wexp) + (int64_t)rg * a.NC * kLanes + lane;
  const uint8_t *sbase = wexp + a.scales_off;
  const int64_t sidx0 = (int64_t)rg * nblk * kLanes + lane;
  uint4 cw[BPW * CPB];
  uint32_t sv[BPW];
  auto load_batch = [&](int g0) __attribute__((always_inline)) {
    static_for<BPW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int b = min(g0 + i, b1 - 1);  // past the end: reload the last block (unused)
      static_for<CPB>([&](auto cc) {
        constexpr int ci = decltype(cc)::value;
        cw[i * CPB + ci] = cptr[((int64_t)b * CPB + ci) * kLanes];
      });
      if constexpr (TR::kAffine)
        sv[i] = reinterpret_cast<const uint32_t *>(sbase)[sidx0 + (int64_t)b * kLanes];
      else
        sv[i] = reinterpret_cast<const uint16_t *>(sbase)[sidx0 + (int64_t)b * kLanes];
    });
  };
  load_batch(b0);

  auto in_row = [&](int m) -> int64_t {
    if (a.dense_M > 0) return m;
    const int p = pbase + m;
    return a.in_gather_token ? (int64_t)a.token_of[p] : (int64_t)p;
  };

  // ---- 2. prologue (overlaps the loads): C and X per row and block, and the
  //         staged activations.  Row offsets come from scalar loads and every
  //         thread of the workgroup takes items, several loads in flight each.
  int64_t rowoff[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) rowoff[m] = (m < M ? in_row(m) : 0) * a.in_row_pairs;
  {
    const int nsum = M * nblk * 16;
#pragma unroll 4
    for (int idx = threadIdx.x; idx < nsum; idx += blockDim.x) {
      const int sub = idx & 15, pm = idx >> 4;
      const int m = pm / nblk, blk = pm - m * nblk;
      int64_t roff = rowoff[0];
#pragma unroll
      for (int mm = 1; mm < MMAX; ++mm) roff = (m == mm) ? rowoff[mm] : roff;
      const int k0 = blk * BLOCK + sub * EPT;
      float cs = 0.f, xs = 0.f;
#pragma unroll
      for (int part = 0; part < PARTS; ++part) {
        const uint32_t *xr = a.in + roff + part * a.in_part_stride + k0 / 2;
        uint32_t xv[EPT / 2];
        uint32_t *xs_l = s_x + (part * MMAX + m) * Kp + k0 / 2;
        if constexpr (EPT == 8) {
          const uint4 v = *reinterpret_cast<const uint4 *>(xr);
          xv[0] = v.x; xv[1] = v.y; xv[2] = v.z; xv[3] = v.w;
          if constexpr (XLDS) *reinterpret_cast<uint4 *>(xs_l) = v;
        } else {
          const uint2 v = *reinterpret_cast<const uint2 *>(xr);
          xv[0] = v.x; xv[1] = v.y;
          if constexpr (XLDS) *reinterpret_cast<uint2 *>(xs_l) = v;
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          const float x = half_to_f32<F16>((xv[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
          const int j = ((k0 + i) % CD::kPeriod) >> 1;
          cs = fmaf(CD::base(j) + (float)TR::kZeroPoint, x, cs);
          xs += x;
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
  const uint32_t *xrow[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) xrow[m] = a.in + rowoff[m];
  __syncthreads();

  // ---- 3. consume batches of BPW blocks
  float acc[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) acc[m] = 0.f;
  const bool sf16 = a.sdtype == QMOE_DTYPE_F16;
  auto consume = [&](int g0) __attribute__((always_inline)) {
    static_for<BPW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int b = g0 + i;
      if (b < b1) {
        float D[MMAX];
#pragma unroll
        for (int m = 0; m < MMAX; ++m) D[m] = 0.f;
        static_for<CPB>([&](auto cc) {
          constexpr int ci = decltype(cc)::value;
          const uint4 wv = cw[i * CPB + ci];
          const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
          const int64_t kp0 = ((int64_t)b * CPB + ci) * PPC;
          static_for<4>([&](auto dc) {
            constexpr int dd = decltype(dc)::value;
            uint32_t pr[PPD];
            CD::extract(wd[dd], pr);
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
              if (m < M) {
                float d = D[m];
#pragma unroll
                for (int part = 0; part < PARTS; ++part) {
                  uint32_t xv[PPD];
                  if constexpr (XLDS) {
                    // same address in every lane: LDS broadcast
                    const uint4 *xl =
                        reinterpret_cast<const uint4 *>(s_x + (part * MMAX + m) * Kp + kp0 + dd * PPD);
#pragma unroll
                    for (int q = 0; q < PPD / 4; ++q) {
                      const uint4 v = xl[q];
                      xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
                    }
                  } else {
                    const uint32_t *xp = xrow[m] + kp0 + dd * PPD + part * a.in_part_stride;
#pragma unroll
                    for (int q = 0; q < PPD; ++q) xv[q] = xp[q];
                  }
#pragma unroll
                  for (int j = 0; j < PPD; ++j) d = dot2<F16>(pr[j], xv[j], d);
                }
                D[m] = d;
              }
            }
          });
        });
        const uint32_t sbits = sv[i];
        const float s = sf16 ? f16_to_f32(sbits & 0xFFFFu) : bf16_to_f32(sbits & 0xFFFFu);
        float bias = 0.f;
        if constexpr (TR::kAffine) bias = sf16 ? f16_to_f32(sbits >> 16) : bf16_to_f32(sbits >> 16);
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
          if (m < M) {
            const float2 cx = reinterpret_cast<const float2 *>(s_corr)[m * nblk + b];
            acc[m] = fmaf(s, D[m] - cx.x, acc[m]);
            if constexpr (TR::kAffine) acc[m] = fmaf(bias, cx.y, acc[m]);
          }
        }
      }
    });
  };
  for (int g0 = b0;;) {
    consume(g0);
    g0 += BPW;
    if (g0 >= b1) break;
    load_batch(g0);
  }

  // ---- 4. cross-wave reduction in a fixed order, then the epilogue
#pragma unroll
  for (int m = 0; m < MMAX; ++m)
    if (m < M) s_red[(wave * MMAX + m) * kLanes + lane] = acc[m];
  __syncthreads();
  const int64_t N = a.N;
  for (int t = threadIdx.x; t < M * kLanes; t += blockDim.x) {
    const int m = t / kLanes, l = t & (kLanes - 1);
    float v = 0.f;
    for (int w = 0; w < KS; ++w) v += s_red[(w * MMAX + m) * kLanes + l];
    const int64_t n = (int64_t)rg * kRowsPerGroup + l;
    if constexpr (EPI == kEpiStoreAct) {
      a.out_act[(int64_t)m * N + n] = f32_to_act(v, a.act_dtype == QMOE_DTYPE_F16);
    } else if constexpr (EPI == kEpiSwiGLU) {
      // rows 2i (gate) and 2i+1 (up) sit in neighbouring lanes
      const float up = __shfl_xor(v, 1);
      if ((l & 1) == 0) {
        const float g = v;
        const float h = g / (1.f + expf(-g)) * up;
        const int64_t Ih = N / 2;
        const int64_t i = (int64_t)rg * (kRowsPerGroup / 2) + (l >> 1);
        const int64_t p = pbase + m;
        const uint16_t hi = f32_to_bf16_rne(h);
        a.h_hi[p * Ih + i] = hi;
        a.h_lo[p * Ih + i] = f32_to_bf16_rne(h - bf16_to_f32(hi));
        if (a.h_dbg) a.h_dbg[(int64_t)a.row_list[p] * Ih + i] = h;
      }
    } else {
      if (a.top_k == 1) {
        // one expert per token: y = w * o straight away (w = 1)
        const int tok = a.token_of[pbase + m];
        a.out_act[(int64_t)tok * N + n] =
            f32_to_act(fmaf(a.route_w[tok], v, 0.f), a.act_dtype == QMOE_DTYPE_F16);
      } else {
        a.out_f32[(int64_t)(pbase + m) * N + n] = v;
      }
    }
  }
}

template <int QT, bool F16, int EPI, int MMAX>
hipError_t launch_gemv_block(const GemvArgs &a, int block, int waves, int grid_slots,
                             hipStream_t s) {
  const dim3 grid((unsigned)(grid_slots * a.RG));
  const dim3 thr((unsigned)(waves * kLanes));
  const size_t lds = gemv_lds_bytes(MMAX, a.nblk, waves, a.K, EPI == kEpiDown ? 2 : 1);
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
  if (epilogue == kEpiDown)
    return launch_gemv_m<QT, false, kEpiDown>(a, block, mmax, waves, grid_slots, s);
  if (epilogue == kEpiSwiGLU)
    return in_f16 ? launch_gemv_m<QT, true, kEpiSwiGLU>(a, block, mmax, waves, grid_slots, s)
                  : launch_gemv_m<QT, false, kEpiSwiGLU>(a, block, mmax, waves, grid_slots, s);
  return in_f16 ? launch_gemv_m<QT, true, kEpiStoreAct>(a, block, mmax, waves, grid_slots, s)
                : launch_gemv_m<QT, false, kEpiStoreAct>(a, block, mmax, waves, grid_slots, s);
}

}  // namespace qmoe
