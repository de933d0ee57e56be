// grouped_impl.hpp -- grouped larger-M path: tiles of 128 routed rows (64 for
// affine formats) x 128 or 256 outputs per workgroup, MFMA
// (v_mfma_f32_16x16x32_f16) on weights dequantized once per tile in registers.
//
// The pages' prefill path runs a grouped GEMM over the rows of each expert
// that dequantizes each weight tile once instead of materialising dense
// experts (onnxruntime pull request 33005, Description: no full A16 expert
// weights; onnx-genai pull request 1167: the grouped M>1 path dequantizes
// once).  The MLX issue 3852 discussion of a small-M tile (BM = 8/16) for the
// M in [10, 32] range is the dense counterpart served by the same kernel.
//
// gfx950 mapping:
//   - a weight code q and its block scale s become one exact f16 value
//     q * s * 2^e: an 8-bit (bf16) significand times a code of at most 3
//     significant bits fits the 11-bit f16 significand, and the per-expert
//     power of two 2^e keeps every product a normal f16 (|q s 2^e| < 2^15).
//     So the fp32 MFMA accumulators run over all of K with no per-block
//     scale epilogue; 2^-e is removed exactly at the end.  An f16 scale
//     (11 bits) times a multi-bit code is split into an 8-bit head and its
//     tail, two exact f16 weights and two MFMAs.  Affine codes are recentred
//     to q = u - 2^(b-1) (INT2: single-bit values) and the recentred bias
//     b + 2^(b-1) s meets per-row block sums of x in the epilogue.
//   - activations are staged in LDS as f16 with a per-row power of two
//     (x * 2^r < 2^14): exact for bf16/f16 x; the fp32 SwiGLU output h is
//     split into f16 hi + lo parts (about 22 significant bits) and FC2 runs
//     one MFMA per part against the same dequantized weights (a single f16
//     h flips too many bf16 output roundings for the tolerance).
//   - the k-tiles run as a two-stage pipeline: the next tile's weights,
//     scales and activations are loaded during the current tile's MFMAs,
//     and the staged activation buffers alternate (one barrier per tile).
//   - B fragments are read straight from the k-tiled prepacked layout: lane
//     l of a wave reads dword (l / 16) of row (l % 16) of a 16-row slice,
//     which that layout stores in the lane's own 16 B; for 2-bit codes a
//     dword holds 16 consecutive k, split over two MFMA k-steps with the A
//     operand gathered in the same k order.
//   - workgroup ids are remapped so that the tiles sharing one expert's
//     weight slice run on the same XCD (its own L2).
#pragma once

#include <float.h>

#include <type_traits>

#include "codec.hpp"
#include "gemv_impl.hpp"
#include "qmoe_internal.h"

namespace qmoe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// Power of two p with amax * p < 2^lim (1 for amax = 0 or non-finite).
__device__ inline float pow2_below(float amax, int lim) {
  if (!(amax > 0.f) || !(amax <= FLT_MAX)) return 1.f;
  int e;
  frexpf(amax, &e);  // amax < 2^e
  int s = lim - e;
  s = max(-120, min(120, s));
  return ldexpf(1.f, s);
}

// ---------------------------------------------------------------- GEMM
// Waves per SIMD (the second launch bound) the 128-row kernels are compiled
// for, which bounds their registers: 16-bit input rows 4 (128 registers);
// split scales (two weight fragments) 2; fp32 rows (two parts) 4 for FC2,
// whose 8-wave workgroups of 2 column slices a wave fit 4 a SIMD by LDS (a
// few registers spill, measured faster than 2 waves a SIMD), and 2 for FC1.
#ifndef QMOE_GROUPED_F32_WAVES
#define QMOE_GROUPED_F32_WAVES 2
#endif
__host__ __device__ constexpr int grouped_waves_per_simd(bool in_f32, bool split, bool fc2) {
  return split ? 2 : !in_f32 ? 4 : fc2 ? 4 : QMOE_GROUPED_F32_WAVES;
}
// Cross-lane moves within 16-lane rows (DPP): quad_perm [1,0,3,2] (lane ^ 1),
// quad_perm [2,3,0,1] (lane ^ 2), and rotations by 4 and 8 lanes.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// SwiGLU epilogue of FC1 (gate and up in neighbouring columns, so in
// neighbouring lanes).  A lane holds rows 4g + {0..3} of its column; the
// even lane of a pair keeps the gates of rows 4g + {0, 1} and takes the ups
// from its partner, the odd lane takes the gates of rows 4g + {2, 3}: every
// lane evaluates two SwiGLUs.  The per-row maximum of |h| (for FC2's row
// scale) is reduced over the 8 lanes of one parity in the 16-lane row, and
// its lanes' maximum goes into the workgroup's per-row maximum in LDS.  The
// SwiGLU itself uses the hardware exponential and reciprocal (about 1 ulp
// each, far below the f16 hi + lo precision FC2 reads h with).
template <int NI, int NJ>
__device__ inline void swiglu_epilogue(const GroupedArgs &a, const floatx4_t (&acc)[NI][NJ], const float *s_rinv,
                                       uint32_t *s_hmax, float winv, const float (&bv)[NJ], int rows, bool wave_on,
                                       int p0, int nw, int lane) {
  const bool odd = lane & 1;
  const int g = lane >> 4;
  const int64_t Ih = a.N / 2;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float inv[4];
#pragma unroll
    for (int el = 0; el < 4; ++el) {
      const int m = 16 * i + 4 * g + el;
      inv[el] = (m < rows && wave_on) ? winv * s_rinv[m] : 0.f;
    }
    const int mr = 16 * i + 4 * g + 2 * (lane & 1);  // this lane's two rows: mr, mr + 1
    const bool v0 = mr < rows && wave_on, v1 = mr + 1 < rows && wave_on;
    float hm0 = 0.f, hm1 = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float v[4];
#pragma unroll
      for (int el = 0; el < 4; ++el) v[el] = fmaf(acc[i][j][el], inv[el], bv[j]);
      const float r0 = dpp_f<kDppXor1>(odd ? v[0] : v[2]);
      const float r1 = dpp_f<kDppXor1>(odd ? v[1] : v[3]);
      const float g0 = odd ? r0 : v[0], g1 = odd ? r1 : v[1];
      const float u0 = odd ? v[2] : r0, u1 = odd ? v[3] : r1;
      const float h0 = a.sw_custom ? swiglu_cfg(g0, u0, a.sw_alpha, a.sw_beta, a.sw_limit)
                                   : g0 * __builtin_amdgcn_rcpf(1.f + __expf(-g0)) * u0;
      const float h1 = a.sw_custom ? swiglu_cfg(g1, u1, a.sw_alpha, a.sw_beta, a.sw_limit)
                                   : g1 * __builtin_amdgcn_rcpf(1.f + __expf(-g1)) * u1;
      const int64_t col = (nw + 16 * j + (lane & 15)) >> 1;
      if (v0) {
        a.out_f32[(int64_t)(p0 + mr) * Ih + col] = h0;
        if (a.h_dbg) a.h_dbg[(int64_t)a.row_list[p0 + mr] * Ih + col] = h0;
        hm0 = fmaxf(hm0, fabsf(h0));
      }
      if (v1) {
        a.out_f32[(int64_t)(p0 + mr + 1) * Ih + col] = h1;
        if (a.h_dbg) a.h_dbg[(int64_t)a.row_list[p0 + mr + 1] * Ih + col] = h1;
        hm1 = fmaxf(hm1, fabsf(h1));
      }
    }
    hm0 = fmaxf(hm0, dpp_f<kDppXor2>(hm0));
    hm1 = fmaxf(hm1, dpp_f<kDppXor2>(hm1));
    hm0 = fmaxf(hm0, dpp_f<kDppRor4>(hm0));
    hm1 = fmaxf(hm1, dpp_f<kDppRor4>(hm1));
    hm0 = fmaxf(hm0, dpp_f<kDppRor8>(hm0));
    hm1 = fmaxf(hm1, dpp_f<kDppRor8>(hm1));
    if ((lane & 14) == 0) {
      if (v0) atomicMax(&s_hmax[mr], __float_as_uint(hm0));
      if (v1) atomicMax(&s_hmax[mr + 1], __float_as_uint(hm1));
    }
  }
}

// s_waitcnt immediate of gfx9: vmcnt 0, expcnt and lgkmcnt at their maxima
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kMaxAffineBlocks = kGroupedMaxAffineBlocks;

// Input modes: 16-bit rows (bf16 or f16) scaled while staged, fp32 rows
// split into f16 hi + lo while staged, f16 rows already scaled (copied), or
// fp32 rows already split into scaled f16 hi + lo parts (copied; a row holds
// the parts of each 8 k together, [hi 8][lo 8], see split_rows_kernel).
enum { kInBf16 = 0, kInF16 = 1, kInF32 = 2, kInScaled = 3, kInSplit = 4 };

// MI: 16-row MFMA row tiles per wave (tile rows TM = 16 MI).  MI = 8 halves
// the LDS reads and the weight dequantization per MFMA of MI = 4: every
// dequantized B fragment feeds 8 row tiles and every A fragment 4 column
// slices; affine formats keep MI = 4 (their per-row block sums need LDS).
// SPLIT: f16 scales of a multi-bit format, split into a head and a tail
// (two MFMAs per weight fragment); an instance of its own, so the common
// case keeps no registers for the tail.
template <int QT, int EPI, int INM, int MI, int NJ, int KT, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW, MI == 8 ? grouped_waves_per_simd(INM == 2, SPLIT, EPI == kGEpiStoreF32) : 1) void grouped_kernel(
    const GroupedArgs a) {
  constexpr bool IN_F32 = INM == kInF32, IN_F16 = INM == kInF16, PRE = INM == kInScaled, SPL = INM == kInSplit;
  using TR = QtTraits<QT>;
  using CD = Codec<TR::kBits, true>;
  constexpr int TM = 16 * MI;          // rows per tile
  constexpr int KC = 128 / TR::kBits;  // k per 16-B chunk: 32 (4-bit) or 64 (2-bit)
  constexpr int NPART = (IN_F32 || SPL) ? 2 : 1;  // fp32 input: f16 hi + lo parts (about 22 bits)
  constexpr int CPT = KT / KC;         // chunks per tile
  constexpr int KS = KT / 32;          // MFMA k-steps per tile
  constexpr int APAD = 8;              // row padding of the staged tile (halves)
  constexpr bool AFF = TR::kAffine;
  static_assert(MI == 4 || MI == 8, "row tiles per wave");
  static_assert(NJ == 2 || NJ == 4, "column slices per wave");
  static_assert(KT == 64 || KT == 128, "k per staged tile");
  static_assert(!AFF || (MI == 4 && NW == 4), "affine block sums are laid out for 64-row tiles, 4 threads a row");
  static_assert(NW == 4 || NW == 8 || NW == 16, "waves per workgroup");
  constexpr int NT = 64 * NW;          // threads per workgroup
  // codes enter the MFMA as q = u - zc: the symmetric codes, and affine codes
  // recentred to [-2^(b-1), 2^(b-1)-1] (bias b + zc*s added in the epilogue)
  constexpr int ZC = AFF ? (1 << (TR::kBits - 1)) : TR::kZeroPoint;
  // codes of more than one significant bit times an 11-bit (f16) scale do not
  // fit f16: the scale is split into an 8-bit head and its tail (two MFMAs)
  constexpr bool MULTIBIT = (QT == QMOE_QTYPE_SYM_INT4 || QT == QMOE_QTYPE_AFFINE_INT4);

  // DIRECT: pre-scaled 16-bit rows or parts (a plain copy) are loaded
  // straight into LDS (global_load_lds, 16 B a lane) into two separate
  // arrays; the other modes convert in registers and store into sA
  constexpr bool DIRECT = (PRE || SPL) && !AFF;
  static_assert(!(SPL && AFF), "pre-split rows feed the non-affine formats only");
  __shared__ _Float16 sA[DIRECT ? 1 : 2][NPART][DIRECT ? 1 : TM][DIRECT ? 1 : KT + APAD];
  __shared__ __attribute__((aligned(16))) _Float16 sD0[DIRECT ? NPART * TM * KT : 8];
  __shared__ __attribute__((aligned(16))) _Float16 sD1[DIRECT ? NPART * TM * KT : 8];
  __shared__ int s_row[TM];
  __shared__ float s_rsc[TM];
  __shared__ float s_rinv[TM];  // 1 / s_rsc (exact: powers of two), 0 past the rows
  __shared__ uint32_t s_hmax[EPI == kGEpiSwiGLU ? TM : 1];  // SwiGLU: the workgroup's max |h| bits per row
  __shared__ float s_X[AFF ? TM : 1][AFF ? kMaxAffineBlocks : 1];  // per-row block sums of x

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int TW = NW * 16 * NJ;  // outputs per tile
  const int ntn = (int)((a.N + TW - 1) / TW);

  // XCD-aware order: blocks are dealt round-robin to the 8 XCDs.  The work
  // items (row tile, column tile) run row-tile major, and each XCD takes a
  // contiguous eighth of them: the column tiles of one row tile run together
  // on one XCD, so its L2 serves the staged activation rows to all of them
  // (and the weights to the next row tile of the same expert).  The grid
  // holds the upper bound of routed tiles; blocks past the actual number exit.
  const int G = gridDim.x;
  const int ntiles = a.dense_M > 0 ? G / ntn : a.tile_info[0].w;
  const int total = ntiles * ntn;
  int bid;
  if (G % 8 == 0) {
    const int chunk = (total + 7) / 8;
    const int r = (int)(blockIdx.x / 8);
    bid = r < chunk ? (int)(blockIdx.x % 8) * chunk + r : total;
  } else {
    bid = (int)blockIdx.x;
  }
  if (bid >= total) return;
  const int tile = bid / ntn, nt = bid - tile * ntn;

  int e, p0, rows;
  if (a.dense_M > 0) {
    e = 0;
    p0 = tile * TM;
    rows = min(TM, a.dense_M - p0);
  } else {
    const int4 ti = a.tile_info[tile];
    e = ti.x;
    p0 = ti.y;
    rows = ti.z;
  }
  if (rows <= 0) return;

  if (threadIdx.x < TM) {
    const int r = threadIdx.x;
    int inrow = -1;
    float sc = 0.f;
    if (r < rows) {
      const int p = p0 + r;
      inrow = (a.dense_M > 0) ? p : (a.in_gather_token ? a.token_of[p] : p);
      sc = (IN_F32 || SPL) ? pow2_below(__uint_as_float(a.in_rowmax[inrow]), 14) : a.in_rowsc[inrow];
    }
    s_row[r] = inrow;
    s_rsc[r] = sc;
    s_rinv[r] = sc > 0.f ? 1.f / sc : 0.f;
    if constexpr (EPI == kGEpiSwiGLU) s_hmax[r] = 0u;
  }
  __syncthreads();

  const float wsc = a.wsc[e];
  const int nw = nt * TW + wave * 16 * NJ;  // first output row of this wave
  const bool wave_on = nw < a.N;           // N not a multiple of the tile: the last tile's upper waves idle
  const int64_t rg = (wave_on ? nw : 0) / kRowsPerGroup;
  const int nl0 = nw % kRowsPerGroup;
  const uint8_t *wexp = a.w + (int64_t)e * a.expert_stride;
  // row group base of the k-tiled layout: [NKT][4 n-tiles][64 lanes][4 dwords]
  const uint32_t *wbase = reinterpret_cast<const uint32_t *>(wexp) + rg * a.NKT * (4 * kLanes * 4);
  const uint8_t *sbase = wexp + a.scales_off;
  // buffer descriptors of this row group's codes and scales: the lane part of
  // each address is fixed per slice, the k-tile part is uniform (soffset)
  constexpr int SES = AFF ? 4 : 2;  // bytes per scale entry
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wbase, (uint32_t)(a.NKT * (4 * kLanes * 16)));
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(sbase + rg * a.NKT * kLanes * a.bpk * SES, (uint32_t)(a.NKT * kLanes * a.bpk * SES));
  const int g = lane >> 4;
  int nl[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) nl[j] = nl0 + 16 * j + (lane & 15);
  // dword g of the chunk of row nl[j] sits in lane (nl[j] % 16) + 16 g of
  // n-tile nl[j] / 16; nl0 is a multiple of 16, so slice j adds the uniform
  // j n-tiles (codes) or 16 j rows (scales) to the first slice's offset
  const int wvo = ((nl0 >> 4) * kLanes + lane) * 16;
  const int svo = nl[0] * a.bpk * SES;
  const bool sf16 = a.sdtype == QMOE_DTYPE_F16;
  constexpr bool split = SPLIT;
  static_assert(!SPLIT || MULTIBIT, "only multi-bit codes split the scale");

  // The whole k loop and epilogue run for NI row tiles: the fewest of MI,
  // MI / 2, ... that hold the tile's rows, chosen once per tile (so the MFMA
  // sequence has no branches and each row tile's A fragment is read while
  // the previous row tile's MFMAs run).
  auto body = [&](auto ni_c) __attribute__((always_inline)) {
    constexpr int NI = decltype(ni_c)::value;
    floatx4_t acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // staging assignment: TPR threads per row, KT/TPR consecutive k each
    constexpr int TPR = NT / TM;
    constexpr int SEG = KT / TPR;
    const int st_r = threadIdx.x / TPR, st_k = (threadIdx.x % TPR) * SEG;
    const int st_in = s_row[st_r];
    const float st_sc = s_rsc[st_r];

    // raw activations of one tile for this thread: SEG values in 16-B pieces
    constexpr int SV = SEG * (IN_F32 ? 4 : 2) / 16;
    auto stage_load = [&](int64_t kt, uint4 (&S)[SV]) __attribute__((always_inline)) {
      if (st_in >= 0 && kt + st_k < a.K) {
        const uint4 *src =
            IN_F32 ? reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(a.in) +
                                                     (int64_t)st_in * a.in_row_elems + kt + st_k)
                   : reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.in) +
                                                     (int64_t)st_in * a.in_row_elems + kt + st_k);
#pragma unroll
        for (int q = 0; q < SV; ++q) S[q] = src[q];
      }
    };
    // scaled f16 into LDS buffer `buf` (zeros past the rows or past K), and
    // the affine block sums of the scaled values
    auto stage_store = [&](int64_t kt, const uint4 (&S)[SV], int buf) __attribute__((always_inline)) {
      // every load of the tile has arrived (the weights were issued first), on
      // every path: the compiler's wait counting then knows that nothing is
      // in flight when the next k-tile's compute() reads the weight registers
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      // 16-B LDS stores of 8 converted values each
      half8_t *dst = reinterpret_cast<half8_t *>(&sA[buf][0][st_r][st_k]);
      half8_t *dlo = reinterpret_cast<half8_t *>(&sA[buf][NPART - 1][st_r][st_k]);
      float xsum = 0.f;
      if (st_in >= 0 && kt + st_k < a.K) {
        if constexpr (IN_F32) {
#pragma unroll
          for (int q = 0; q < SV / 2; ++q) {
            half8_t hv, lv;
#pragma unroll
            for (int h = 0; h < 8; ++h) {
              const uint4 &v = S[2 * q + h / 4];
              const uint32_t w = (h % 4 == 0) ? v.x : (h % 4 == 1) ? v.y : (h % 4 == 2) ? v.z : v.w;
              const float xs = __uint_as_float(w) * st_sc;
              const _Float16 hi = (_Float16)xs;
              hv[h] = hi;
              lv[h] = (_Float16)(xs - (float)hi);
              xsum += xs;
            }
            dst[q] = hv;
            dlo[q] = lv;
          }
        } else if constexpr (PRE) {
#pragma unroll
          for (int q = 0; q < SV; ++q) {
            const half8_t hv = __builtin_bit_cast(half8_t, S[q]);
            dst[q] = hv;
            if constexpr (AFF) {
#pragma unroll
              for (int h = 0; h < 8; ++h) xsum += (float)hv[h];
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < SV; ++q) {
            const uint32_t wv[4] = {S[q].x, S[q].y, S[q].z, S[q].w};
            half8_t hv;
#pragma unroll
            for (int h = 0; h < 8; ++h) {
              const uint32_t bits = (wv[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
              const float xs = half_to_f32<IN_F16>(bits) * st_sc;
              hv[h] = (_Float16)xs;
              xsum += xs;
            }
            dst[q] = hv;
          }
        }
      } else {
        const half8_t z = {};
#pragma unroll
        for (int q = 0; q < SEG / 8; ++q) {
          dst[q] = z;
          if constexpr (NPART == 2) dlo[q] = z;
        }
      }
      if constexpr (AFF) {
        // the 4 threads of a row hold 4 consecutive SEG-k segments; blocks are
        // 64 or 128 k: a block inside the tile (64 < KT) sums 2 threads, a
        // block spanning tiles (block >= KT) sums all 4 and is written by its
        // first tile and added by the next (same thread, in order)
        const float p1 = xsum + __shfl_xor(xsum, 1);
        const float p2 = p1 + __shfl_xor(p1, 2);
        if (kt + st_k < a.K) {
          if (a.block < KT) {
            if ((threadIdx.x & 1) == 0) s_X[st_r][(kt + st_k) / a.block] = p1;
          } else if ((threadIdx.x & 3) == 0) {
            float &d = s_X[st_r][kt / a.block];
            d = (kt % a.block == 0) ? p2 : d + p2;
          }
        }
      }
    };
    // weight dwords and scales of one tile (a partial last tile re-reads the
    // last chunk; its A columns are zero)
    // chunk -> scale entry without divisions: a k-tile holds 4 chunks, and
    // blocks x chunks-per-block = 4, so the k-tile of chunk c is c >> 2 and
    // its block within the k-tile is (c >> log2(chunks per block)) & (bpk - 1)
    const int cpb_log = __builtin_ctz((unsigned)(a.block / KC));
    const int bpk = a.bpk;
    // scale entries stay 16-bit until compute() widens them: a widening at the
    // load would make the loop wait for the prefetched scales at once
    using ST = std::conditional_t<AFF, uint32_t, uint16_t>;
    auto load_b = [&](int64_t kt, uint32_t (&bw)[CPT][NJ], ST (&sv)[CPT][NJ]) __attribute__((always_inline)) {
      if constexpr (CPT == 2 && !AFF) {
        // a tile of two chunks: its first chunk is even, so both sit in one
        // 8-B half of the lane's 16 B (a partial last tile reads the padding
        // chunk beside it; its A columns are zero), and one scale serves both
        // chunks when a block spans two or more
        const int chunk = (int)(kt / KC);
        const int ktile = chunk >> 2, bi0 = (chunk >> cpb_log) & (bpk - 1);
        const int wso = ktile * (4 * kLanes * 16) + (chunk & 3) * 4;
        const int sso = (ktile * kLanes * bpk + bi0) * SES;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int wj = wso + j * (kLanes * 16), sj = sso + j * 16 * bpk * SES;
          const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(wrs, wvo, wj, 0);
          bw[0][j] = w2[0];
          bw[1][j] = w2[1];
          sv[0][j] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo, sj, 0);
        }
        if (cpb_log == 0) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            sv[1][j] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo, sso + SES + j * 16 * bpk * SES, 0);
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j) sv[1][j] = sv[0][j];
        }
        return;
      }
      static_for<CPT>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const int chunk = min((int)(kt / KC) + c, (int)a.NC - 1);
        const int ktile = chunk >> 2, bi = (chunk >> cpb_log) & (bpk - 1);
        const int wso = ktile * (4 * kLanes * 16) + (chunk & 3) * 4;
        const int sso = (ktile * kLanes * bpk + bi) * SES;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int wj = wso + j * (kLanes * 16), sj = sso + j * 16 * bpk * SES;
          bw[c][j] = __builtin_amdgcn_raw_buffer_load_b32(wrs, wvo, wj, 0);
          if constexpr (AFF) sv[c][j] = __builtin_amdgcn_raw_buffer_load_b32(srs, svo, sj, 0);
          else sv[c][j] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo, sj, 0);
        }
      });
    };
    const RegConsts<CD::kNC> dk = CodecOps<CD>::in_registers();  // decoder constants in registers
    // A: part 0 of the staged tile; RS halves between rows, PS between parts;
    // SWZ: 16-B pieces stored at slot piece ^ (row & 7) (the direct layout)
    auto compute = [&](const _Float16 *A, auto rs_c, auto ps_c, auto swz_c, const uint32_t (&bw)[CPT][NJ],
                       const ST (&sv)[CPT][NJ]) __attribute__((always_inline)) {
      constexpr int RS = decltype(rs_c)::value, PS = decltype(ps_c)::value;
      constexpr bool SWZ = decltype(swz_c)::value;
      // per chunk and slice: the pre-scaled f16 scale (head) and its tail,
      // once per tile
      f16x2_t s2c[CPT][NJ], l2c[CPT][NJ];
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const uint32_t sb = sv[c][j];
          const float s = sf16 ? f16_to_f32(sb & 0xFFFFu) : bf16_to_f32(sb & 0xFFFFu);
          // head: s rounded to 8 significant bits; tail: the rest (0 for bf16 scales)
          const float sh = split ? bf16_to_f32(f32_to_bf16_rne(s)) : s;
          const _Float16 shs = (_Float16)(sh * wsc), sls = (_Float16)((s - sh) * wsc);
          s2c[c][j] = f16x2_t{shs, shs};
          l2c[c][j] = f16x2_t{sls, sls};
        }
      static_for<KS>([&](auto kc_) {
        constexpr int ks = decltype(kc_)::value;
        // each k-step's decode stays after the previous k-step's MFMAs: the
        // schedule is kept as written, which bounds the registers in use
        __builtin_amdgcn_sched_barrier(0);
        constexpr int c = ks * 32 / KC;               // chunk of this k-step
        constexpr int half = (ks * 32 % KC) / 32;     // 2-bit: which 8 of the dword's 16 k
        half8_t bf[NJ], bl[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          uint32_t pr[CD::kPairs];
          CD::extract(bw[c][j], pr, dk);
          const f16x2_t s2 = s2c[c][j], l2 = l2c[c][j];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int jj = half * 4 + q;  // pair index within the dword
            const _Float16 off = (_Float16)(CD::base(jj) + (float)ZC);
            const f16x2_t off2 = {off, off};
            const f16x2_t qv = __builtin_bit_cast(f16x2_t, pr[jj]) - off2;  // exact code
            const f16x2_t wh = qv * s2, wl = qv * l2;                       // exact products
            bf[j][2 * q] = wh[0];
            bf[j][2 * q + 1] = wh[1];
            bl[j][2 * q] = wl[0];
            bl[j][2 * q + 1] = wl[1];
          }
        }
        // A fragments: row (lane % 16) of each 16-row slice, 8 k in the order of B
        const int koff = (TR::kBits == 4) ? (ks * 32 + 8 * g) : (c * 64 + 16 * g + 8 * half);
        const int kslot = SWZ ? (((koff >> 3) ^ (lane & 7)) << 3) : koff;  // rows 16 i + r share r & 7
        const _Float16 *abase = A + (lane & 15) * RS + kslot;
        constexpr int PST = PS, RST = 16 * RS;  // halves between parts, row tiles
        // the A fragments of row tile i + AD - 1 are read while row tile i's
        // MFMAs run, and scheduling fences keep that order, so at most AD
        // fragments (per part) are held in registers
        constexpr int AD = (NPART == 1 && MI == 8) ? QMOE_GROUPED_AD16 : QMOE_GROUPED_AD;
        half8_t af[AD][NPART];
        auto read_a = [&](int i, half8_t(&d)[NPART]) __attribute__((always_inline)) {
#pragma unroll
          for (int pp = 0; pp < NPART; ++pp) d[pp] = *reinterpret_cast<const half8_t *>(abase + i * RST + pp * PST);
        };
        static_for<(NI < AD - 1 ? NI : AD - 1)>([&](auto ic) { read_a(decltype(ic)::value, af[decltype(ic)::value]); });
        static_for<NI>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i + AD - 1 < NI) read_a(i + AD - 1, af[(i + AD - 1) % AD]);
#pragma unroll
          for (int pp = 0; pp < NPART; ++pp)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i % AD][pp], bf[j], acc[i][j], 0, 0, 0);
              if (split) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i % AD][pp], bl[j], acc[i][j], 0, 0, 0);
            }
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    };

    // Two-stage pipeline over the k-tiles: the next tile's weights, scales and
    // activations are loaded while the current one is multiplied; one barrier
    // per tile (the staged buffers alternate).
    uint32_t bwA[CPT][NJ], bwB[CPT][NJ];
    ST svA[CPT][NJ], svB[CPT][NJ];
    if constexpr (DIRECT) {
      // Each wave copies IPW blocks of 1 KiB (RPI rows) per tile: lane l
      // takes piece slot l % PPR of row l / PPR, and reads the row's global
      // piece slot ^ (row & 7).  Rows past the tile read token row 0 (their
      // outputs are never stored); pieces past K are cleared after the copy.
      constexpr int PPR = KT / 8, RPI = kLanes / PPR, IPW = TM / RPI / NW;
      static_assert(TM % (RPI * NW) == 0, "direct copy blocks");
      const uint16_t *gsrc[IPW];
      int dslot[IPW];
#pragma unroll
      for (int q = 0; q < IPW; ++q) {
        const int row = (q * NW + wave) * RPI + lane / PPR, slot = lane % PPR;
        const int in = s_row[row];
        gsrc[q] = reinterpret_cast<const uint16_t *>(a.in) + (int64_t)(in >= 0 ? in : 0) * a.in_row_elems;
        dslot[q] = (slot ^ (row & 7)) * 8;  // k of this lane's piece within the tile
      }
      // a piece past K reads the row's last 8 values instead (K >= 32); a
      // pre-split row holds [hi 8][lo 8] per 8 k, part p of the piece at k
      // at 2 k + 8 p, and part p lands TM x KT halves after part 0
      constexpr int KM = SPL ? 2 : 1;
      auto dma = [&](int64_t kt, _Float16 *D) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < IPW; ++q) {
          const int64_t k = kt + dslot[q] < a.K - 8 ? kt + dslot[q] : a.K - 8;
#pragma unroll
          for (int pp = 0; pp < NPART; ++pp)
            // (untyped pointers: a typed source pointer keeps the host pass from emitting the kernel's stub)
            __builtin_amdgcn_global_load_lds((const void *)(gsrc[q] + KM * k + 8 * pp),
                                             (void *)(D + pp * TM * KT + (q * NW + wave) * RPI * KT), 16, 0, 0);
        }
      };
      // after the copy of the tile at kt has landed: clear its pieces past K
      auto clear_tail = [&](int64_t kt, _Float16 *D) __attribute__((always_inline)) {
        if (kt + KT > a.K) {
#pragma unroll
          for (int q = 0; q < IPW; ++q)
            if (kt + dslot[q] >= a.K)
#pragma unroll
              for (int pp = 0; pp < NPART; ++pp)
                *reinterpret_cast<uint4 *>(D + pp * TM * KT + (q * NW + wave) * RPI * KT + lane * 8) =
                    make_uint4(0u, 0u, 0u, 0u);
        }
      };
      using RSc = std::integral_constant<int, KT>;
      using PSc = std::integral_constant<int, TM * KT>;
      using SWc = std::integral_constant<bool, true>;
      load_b(0, bwA, svA);
      dma(0, sD0);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      clear_tail(0, sD0);
      __syncthreads();
      for (int64_t kt = 0; kt < a.K; kt += 2 * KT) {
        const bool more0 = kt + KT < a.K;
        if (more0) {
          load_b(kt + KT, bwB, svB);
          dma(kt + KT, sD1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (wave_on) compute(sD0, RSc{}, PSc{}, SWc{}, bwA, svA);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if (!more0) break;
        clear_tail(kt + KT, sD1);
        __syncthreads();
        const bool more1 = kt + 2 * KT < a.K;
        if (more1) {
          load_b(kt + 2 * KT, bwA, svA);
          dma(kt + 2 * KT, sD0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (wave_on) compute(sD1, RSc{}, PSc{}, SWc{}, bwB, svB);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if (more1) clear_tail(kt + 2 * KT, sD0);
        __syncthreads();
      }
    } else {
      uint4 S[SV];
      load_b(0, bwA, svA);
      stage_load(0, S);
      stage_store(0, S, 0);
      __syncthreads();
      int buf = 0;
      for (int64_t kt = 0; kt < a.K; kt += KT) {
        const bool more = kt + KT < a.K;
        if (more) {
          load_b(kt + KT, bwB, svB);
          stage_load(kt + KT, S);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (wave_on)  // uniform: idle waves of a partial last column tile only stage
          compute(&sA[buf][0][0][0], std::integral_constant<int, KT + APAD>{},
                  std::integral_constant<int, TM * (KT + APAD)>{}, std::integral_constant<bool, false>{}, bwA, svA);
        __builtin_amdgcn_sched_barrier(0);
        if (more) stage_store(kt + KT, S, buf ^ 1);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CPT; ++c)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            bwA[c][j] = bwB[c][j];
            svA[c][j] = svB[c][j];
          }
        buf ^= 1;
      }
    }

    // affine: + sum over blocks of (b + zc*s) * X[row][block], scaled like acc
    if constexpr (AFF) {
      if (wave_on) {
        for (int blk = 0; blk < (int)a.nblk; ++blk) {
          float bb[NJ];
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const uint32_t sb = reinterpret_cast<const uint32_t *>(
                sbase)[((rg * a.NKT + blk / a.bpk) * kLanes + nl[j]) * a.bpk + blk % a.bpk];
            const float s = sf16 ? f16_to_f32(sb & 0xFFFFu) : bf16_to_f32(sb & 0xFFFFu);
            const float b = sf16 ? f16_to_f32(sb >> 16) : bf16_to_f32(sb >> 16);
            bb[j] = fmaf((float)ZC, s, b) * wsc;
          }
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int el = 0; el < 4; ++el) {
              const float X = s_X[16 * i + 4 * g + el][blk];
#pragma unroll
              for (int j = 0; j < NJ; ++j) acc[i][j][el] = fmaf(bb[j], X, acc[i][j][el]);
            }
        }
      }
    }

    // epilogue: lane holds rows 16i + 4(lane/16) + el, column 16j + lane%16;
    // the optional per-expert output bias goes in before the SwiGLU or store
    const float winv = 1.f / wsc;
    float bv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      bv[j] = (a.bias && wave_on) ? half_to_f32_rt(a.bias[(int64_t)e * a.N + nw + 16 * j + (lane & 15)],
                                                   a.act_dtype == QMOE_DTYPE_F16)
                                  : 0.f;  // idle waves of a partial last tile read nothing
    if constexpr (EPI == kGEpiSwiGLU) {
      if (!a.relu) {
        swiglu_epilogue<NI, NJ>(a, acc, s_rinv, s_hmax, winv, bv, rows, wave_on, p0, nw, lane);
        // one global atomic per row and workgroup
        __syncthreads();
        if ((int)threadIdx.x < rows) atomicMax(&a.out_rowmax[p0 + threadIdx.x], s_hmax[threadIdx.x]);
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int el = 0; el < 4; ++el) {
        const int m = 16 * i + 4 * g + el;
        const bool valid = m < rows && wave_on;
        const float inv = valid ? winv * s_rinv[m] : 0.f;
        float hmax = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float v = fmaf(acc[i][j][el], inv, bv[j]);
          const int64_t n = nw + 16 * j + (lane & 15);
          if constexpr (EPI == kGEpiSwiGLU) {
            // SwiGLU over neighbouring gate/up lanes, or (a.relu) h = max(a, 0) per row
            const float up = __shfl_xor(v, 1);
            if (valid && (a.relu || (lane & 1) == 0)) {
              const float h = a.relu        ? fmaxf(v, 0.f)
                              : a.sw_custom ? swiglu_cfg(v, up, a.sw_alpha, a.sw_beta, a.sw_limit)
                                            : v / (1.f + expf(-v)) * up;
              const int64_t p = p0 + m;
              const int64_t Ih = a.relu ? a.N : a.N / 2, i = a.relu ? n : n / 2;
              a.out_f32[p * Ih + i] = h;
              if (a.h_dbg) a.h_dbg[(int64_t)a.row_list[p] * Ih + i] = h;
              hmax = fmaxf(hmax, fabsf(h));
            }
          } else if constexpr (EPI == kGEpiStoreF32) {
            if (valid) a.out_f32[(int64_t)(p0 + m) * a.N + n] = v;
          } else {
            if (valid) a.out_act[(int64_t)(p0 + m) * a.N + n] = f32_to_act(v, a.act_dtype == QMOE_DTYPE_F16);
          }
        }
        if constexpr (EPI == kGEpiSwiGLU) {
          // max over the 16 lanes that share row m, then one atomic per row
#pragma unroll
          for (int off = 8; off >= 1; off >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, off));
          if (valid && (lane & 15) == 0) atomicMax(&a.out_rowmax[p0 + m], __float_as_uint(hmax));
        }
      }
    }
  };
  const int mi_on = (rows + 15) >> 4;  // row tiles holding rows of this tile
  if (mi_on > MI / 2) body(std::integral_constant<int, MI>{});
  else if (mi_on > MI / 4) body(std::integral_constant<int, MI / 2>{});
  else if constexpr (MI / 8 >= 1) {
    if (mi_on > MI / 8) body(std::integral_constant<int, MI / 4>{});
    else body(std::integral_constant<int, MI / 8>{});
  } else {
    body(std::integral_constant<int, MI / 4>{});
  }
}


template <int QT, int EPI, bool MAIN, bool SPLIT>
hipError_t launch_grouped_split(const GroupedArgs &a, int grid, hipStream_t s) {
#define QMOE_GK(INM, S) grouped_kernel<QT, EPI, INM, S.mi, S.nj, S.kt, S.nw, SPLIT>, dim3(grid), dim3(64 * S.nw), 0, s, a
  constexpr GroupedShape S16 = MAIN ? grouped_shape_main(false) : grouped_shape_64(false);
  constexpr GroupedShape S32 = MAIN ? grouped_shape_main(true) : grouped_shape_64(true);
  // the inputs each epilogue is used with: FC1 pre-scaled token rows (or
  // fp32 token rows, staged as hi + lo parts), FC2 the fp32 SwiGLU output,
  // the dense matrix 16-bit rows
  if constexpr (EPI == kGEpiSwiGLU) {
    if (a.in_f32)
      return qlaunch(QMOE_GK(kInF32, S16));
    if (!a.in_scaled) return hipErrorInvalidConfiguration;
    return qlaunch(QMOE_GK(kInScaled, S16));
  } else if constexpr (EPI == kGEpiStoreF32) {
    if constexpr (!QtTraits<QT>::kAffine) {
      if (a.in_split) return qlaunch(QMOE_GK(kInSplit, S32));
    }
    if (!a.in_f32 || a.in_split) return hipErrorInvalidConfiguration;
    return qlaunch(QMOE_GK(kInF32, S32));
  } else {
    if (a.in_f32 || a.in_scaled) return hipErrorInvalidConfiguration;
    if (a.in_f16)
      return qlaunch(QMOE_GK(kInF16, S16));
    return qlaunch(QMOE_GK(kInBf16, S16));
  }
#undef QMOE_GK
}

template <int QT, int EPI, bool MAIN>
hipError_t launch_grouped_shape(const GroupedArgs &a, int grid, hipStream_t s) {
  constexpr bool MULTIBIT = QtTraits<QT>::kBits == 4;
  if constexpr (MULTIBIT) {
    if (a.sdtype == QMOE_DTYPE_F16) return launch_grouped_split<QT, EPI, MAIN, true>(a, grid, s);
  }
  return launch_grouped_split<QT, EPI, MAIN, false>(a, grid, s);
}

// The kernel instance of the tile shape grouped_shape gives for the call's
// tile rows (64-row tiles, or the main shape of non-affine formats).
template <int QT, int EPI>
hipError_t launch_grouped_in(const GroupedArgs &a, int grid, hipStream_t s) {
  if constexpr (!QtTraits<QT>::kAffine) {
    if (a.tile_rows == 16 * QMOE_GROUPED_MI)
      return launch_grouped_shape<QT, EPI, true>(a, grid, s);
  }
  if (a.tile_rows != kTileM) return hipErrorInvalidConfiguration;
  return launch_grouped_shape<QT, EPI, false>(a, grid, s);
}

// Launch with the instance of one epilogue for the matrix's format (defined in
// one translation unit per epilogue).
template <int EPI>
hipError_t launch_grouped_epi(const GroupedArgs &a, int grid, hipStream_t s) {
  switch (a.qtype) {
    case QMOE_QTYPE_SYM_INT4: return launch_grouped_in<QMOE_QTYPE_SYM_INT4, EPI>(a, grid, s);
    case QMOE_QTYPE_SYM_INT2: return launch_grouped_in<QMOE_QTYPE_SYM_INT2, EPI>(a, grid, s);
    case QMOE_QTYPE_TERNARY: return launch_grouped_in<QMOE_QTYPE_TERNARY, EPI>(a, grid, s);
    case QMOE_QTYPE_AFFINE_INT2: return launch_grouped_in<QMOE_QTYPE_AFFINE_INT2, EPI>(a, grid, s);
    default: return launch_grouped_in<QMOE_QTYPE_AFFINE_INT4, EPI>(a, grid, s);
  }
}

}  // namespace qmoe
