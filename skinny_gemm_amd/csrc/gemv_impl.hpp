// gemv_impl.hpp -- quantized GEMV for up to 16 rows per expert (32 dense rows)
// on the matrix cores.
//
// Computes out[m][n] = sum_k W[n][k] * in[m][k] for the rows m routed to one
// expert (or M dense rows), dequantizing every weight chunk once in VGPRs and
// applying it to all rows at once.  This is the register-level answer to the
// per-token GEMV problem of the inference-research gotcha page on QMoE (loop
// over the tokens that share an expert inside the kernel instead of one GEMV
// per token) and the fused gate/up SwiGLU expert GEMV + down GEMV of
// onnx-genai pull request 1167.
//
// gfx950 mapping (the pages' designs use one warp or thread group per row):
//   - a wave owns TN n-tiles of 16 output rows (TN = 4: a whole 64-row
//     group; TN = 1 when the grid would otherwise leave compute units idle)
//     and a contiguous run of k-tiles; per k-tile it issues TN 1 KiB
//     contiguous loads (16 B per lane) of the prepacked layout, whose lane
//     (r, g) = (lane % 16, lane / 16) holds exactly the v_mfma_f32_16x16x32 B
//     operand of row r for k-group g, and the next k-tile's loads are in
//     flight during the current one's MFMAs (buffer loads, see the k loop);
//   - one AND-OR per weight pair turns the codes into exact 16-bit floats
//     base + u (magic-number decoding, codec.hpp); the raw codes enter the
//     MFMA unscaled, so the dequantization costs no multiply;
//   - the activations of up to 16 rows are the A operand, read straight from
//     global memory (they are tiny and stay in L2): one tile covers every
//     row of an expert, so rows 2..16 cost matrix-core cycles only;
//   - per block, fresh accumulators D = sum (base + u) x; a second MFMA
//     against a constant B operand gives C = sum (base + zero point) x (and
//     X = sum x for affine formats) in the same lane layout, and the block
//     epilogue adds s (D - C) (+ b X) to the fp32 result;
//   - K is split over the waves of a workgroup; the partial sums meet in LDS
//     and are added in a fixed wave order;
//   - for small decode batches the FC1 launch routes the tokens itself
//     (epilogue kEpiSwiGLURouted): every workgroup runs the top-k and finds
//     its own expert's rows, so no routing kernel precedes it.
#pragma once

#include "codec.hpp"
#include "qmoe_internal.h"
#include "route_impl.hpp"

// Build option: 1 (default) keeps the next k-tile's weights in flight during
// the current one's MFMAs; 0 loads and computes one k-tile at a time.
#ifndef QMOE_GEMV_PREFETCH
#define QMOE_GEMV_PREFETCH 1
#endif


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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_{bf16,f16}: c + A (16 x 32) * B (32 x 16).  Lane l
// supplies row l % 16 of A and column l % 16 of B for k = 8 (l / 16) .. +7;
// it receives C rows 4 (l / 16) + i, i = 0..3, of column l % 16.
template <bool F16>
__device__ inline floatx4_t mfma16(const uint4 &a, const uint4 &b, const floatx4_t &c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16-bit float bits of a small non-negative integer v < 2048 (exact).
template <bool F16>
__host__ __device__ constexpr uint32_t small_int_bits(int v) {
  if (v == 0) return 0;
  int e = 0;
  while ((2 << e) <= v) ++e;  // 2^e <= v < 2^(e+1)
  if (F16) return (uint32_t)(((15 + e) << 10) | ((v - (1 << e)) << (10 - e)));
  return (uint32_t)(((127 + e) << 7) | ((v - (1 << e)) << (7 - e)));
}

// Raw buffer loads for the weight stream.  They are intrinsic calls, not IR
// loads, so the optimiser cannot fold a loop-carried prefetch back into a
// load at the top of the next iteration (which a phi of two plain loads
// invites); the wave-uniform base sits in a buffer descriptor in SGPRs and
// the uniform part of each offset goes in soffset.  Descriptor word 3 is the
// gfx9-family raw-dword format; num_records bounds the region.
constexpr int kBufferWord3 = 0x00020000;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferWord3);
}
__device__ inline uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Scales of one row for one k-tile: BYTES = blocks per k-tile x entry size.
template <int BYTES>
__device__ inline void load_scales(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t (&sv)[4]) {
  if constexpr (BYTES == 16) {
    const uint4 v = buf_load16(r, voff, soff);
    sv[0] = v.x; sv[1] = v.y; sv[2] = v.z; sv[3] = v.w;
  } else if constexpr (BYTES == 8) {
    const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    sv[0] = v.x; sv[1] = v.y; sv[2] = 0; sv[3] = 0;
  } else if constexpr (BYTES == 4) {
    sv[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0); sv[1] = sv[2] = sv[3] = 0;
  } else {
    sv[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0); sv[1] = sv[2] = sv[3] = 0;
  }
}

// QT: code format; XF16: the A operand (and the decoding) is f16, else bf16;
// PARTS: 2 = the input is an fp32 value split into bf16 hi + lo rows;
// MR: accumulator rows kept per lane (1: a single row, 4: up to 16 rows per
// tile); MT: 16-row tiles; BLOCK: scale block along K.
template <int QT, bool XF16, int PARTS, int EPI, int MR, int MT, int BLOCK, int TN, bool EXT>
__global__ __launch_bounds__(EPI == kEpiDownCat ? 64 * kGemvCatMaxWaves : 512) void gemv_kernel(const GemvArgs a) {
  using TR = QtTraits<QT>;
  using CD = Codec<TR::kBits, XF16>;
  constexpr int BITS = TR::kBits;
  constexpr int KC = 128 / BITS;             // k per chunk
  constexpr int KT = 4 * KC;                 // k per k-tile
  constexpr int HALVES = BITS == 2 ? 2 : 1;  // MFMA k-steps per chunk
  constexpr int KSTEPS = 4 * HALVES;         // k-steps per k-tile
  constexpr int CPB = BLOCK / KC;            // chunks per block
  constexpr int BPK = KT / BLOCK;            // blocks per k-tile
  constexpr bool AFF = TR::kAffine;
  constexpr int ESZ = AFF ? 4 : 2;
  constexpr int ZP = TR::kZeroPoint;
  static_assert(CPB >= 1 && BPK >= 1, "block must span whole chunks of one k-tile");
  static_assert(MR == 4 || MT == 1, "several row tiles keep all accumulator rows");
  static_assert(TN == 1 || TN == 2 || TN == 4, "n-tiles per wave");

  extern __shared__ float s_red[];  // [waves][TN][MT][MR][64]
  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int KS = blockDim.x / kLanes;
  // workgroup -> (slot, row group, group of TN n-tiles within the row group)
  constexpr int TQ = 4 / TN;
  const int RG = (int)a.RG;
  const int slot = (int)blockIdx.x / (RG * TQ);
  const int rgq = (int)blockIdx.x - slot * (RG * TQ);
  const int rg = rgq / TQ, t0 = (rgq - rg * TQ) * TN;

  constexpr bool ROUTED = EPI == kEpiSwiGLURouted;
  constexpr bool SWIGLU = EPI == kEpiSwiGLU || ROUTED;
  constexpr bool CAT = EPI == kEpiDownCat;  // one token's k experts as one concatenated K
  // routed: this workgroup's expert and the flat slots of its rows
  __shared__ int32_t s_rslot[ROUTED ? kGemvMaxRows : 1];
  __shared__ int32_t s_ids[ROUTED ? kLanes : 1];  // routed: expert of each flat slot
  int e, M, pbase;
  if (CAT) {
    e = 0;  // per k segment below
    M = 1;
    pbase = 0;
  } else if (a.dense_M > 0) {
    e = 0;
    M = a.dense_M;
    pbase = 0;
  } else if constexpr (ROUTED) {
    // every workgroup routes the (at most 64) slots itself and finds its own
    // expert's entry; workgroup 0 also writes the top-k ids and weights, and
    // the global lists at the end of the kernel (read by later kernels only)
    __shared__ int4 s_slot;
    __shared__ TopkScratch s_tk[kGemvMaxWaves];
    const bool lead = blockIdx.x == 0;
    for (int t = wave; t < a.route_T; t += KS) {
      const float *lt = a.logits + (int64_t)t * a.route_E;
      int32_t *ids_t = lead ? a.route.ids + (int64_t)t * a.route_k : nullptr;
      float *w_t = lead ? a.route.w + (int64_t)t * a.route_k : nullptr;
      // EXT instances also serve the unnormalised top-k weights
      if constexpr (EXT) {
        if (a.route_softmax_all) {
          wave_topk<true>(lt, a.route_E, a.route_k, ids_t, w_t, s_ids + t * a.route_k, &s_tk[wave]);
          continue;
        }
      }
      wave_topk(lt, a.route_E, a.route_k, ids_t, w_t, s_ids + t * a.route_k, &s_tk[wave]);
    }
    __syncthreads();
    if (wave == 0) wave_expand_want(s_ids, a.route_T * a.route_k, slot, &s_slot, s_rslot);
    // workgroup 0: the expert map of all slots for the later kernels (on a
    // wave that is otherwise waiting here, when there is one)
    if (lead && wave == (KS > 1 ? 1 : 0))
      wave_expand_lists(s_ids, a.route_T * a.route_k, a.route_k, a.route_E, a.route_max_slots, a.route);
    __syncthreads();
    const int4 si = s_slot;  // the same for every lane: keep it in SGPRs
    e = __builtin_amdgcn_readfirstlane(si.x);
    M = __builtin_amdgcn_readfirstlane(si.y);
    pbase = __builtin_amdgcn_readfirstlane(si.z);
    if (M <= 0) return;
  } else {
    const int4 si = a.slot_info[slot];
    e = si.x;
    M = si.y;
    pbase = si.z;
    if (M <= 0) return;
  }
  if (M > 16 * MT) M = 16 * MT;  // the host sizes MT for every row count; the clamp keeps accesses in bounds
  const int r = lane & 15, g = lane >> 4;
  const int NKT = (int)a.NKT, NC = (int)a.NC;
  // this wave's k-tiles: of the matrix, or (CAT) of the k matrices end to end
  const int NKW = CAT ? NKT * a.route_k : NKT;
  const int kw0 = (int)((int64_t)wave * NKW / KS), kw1 = (int)((int64_t)(wave + 1) * NKW / KS);
  // CAT: the routing entries of the wave's first matrix, loaded before the
  // set-up below so that their latency overlaps it
  int cat_e0 = 0;
  float cat_w0 = 0.f;
  if constexpr (CAT) {
    const int j0 = min(kw0 / NKT, a.route_k - 1);
    cat_e0 = a.route.ids[j0];
    cat_w0 = a.route.w[j0];
  }

  // A operand rows: lane (r, g) supplies row 16 mt + r.  Rows past M read
  // row 0 instead: an A row only feeds the output row of the same index,
  // which is never stored, so the loads need no per-lane masking.
  const uint32_t *arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m0 = 16 * mt + r;
    const int m = m0 < M ? m0 : 0;
    int64_t row = 0;
    {
      if (CAT) row = 0;  // per k segment below
      else if (a.dense_M > 0) row = m;
      else if constexpr (ROUTED) row = s_rslot[m] / a.route_k;
      else row = a.in_gather_token ? (int64_t)a.token_of[pbase + m] : (int64_t)(pbase + m);
    }
    arow[mt] = a.in + row * a.in_row_pairs;
  }

  // this row group's codes (NKT x 4 KiB) and scales (NKT x 64 rows x BPK
  // entries) of expert e (CAT: reset for each segment's expert)
  auto code_rsrc = [&](int ex) {
    return make_rsrc(a.w + (int64_t)ex * a.expert_stride + (int64_t)rg * NKT * (4 * kLanes * 16),
                     (uint32_t)NKT * (4 * kLanes * 16));
  };
  auto scale_rsrc = [&](int ex) {
    return make_rsrc(a.w + (int64_t)ex * a.expert_stride + a.scales_off + (int64_t)rg * NKT * kLanes * (BPK * ESZ),
                     (uint32_t)NKT * kLanes * (BPK * ESZ));
  };
  __amdgpu_buffer_rsrc_t wrs = code_rsrc(e);
  __amdgpu_buffer_rsrc_t srs = scale_rsrc(e);
  float wseg = 1.f;  // CAT: the routing weight of the segment's expert
  const int wvoff = lane * 16, svoff = r * (BPK * ESZ);
  const uint32_t smask = opaque_v(a.sdtype == QMOE_DTYPE_F16 ? 0xFFFFFFFFu : 0u);

  // constant B operands: (base + zero point) per k position, and ones
  uint4 bc[HALVES];
#pragma unroll
  for (int h = 0; h < HALVES; ++h) {
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t bits = small_int_bits<XF16>((int)CD::base(4 * h + q) + ZP);
      v[q] = bits | (bits << 16);
    }
    bc[h] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  constexpr uint32_t kOne = small_int_bits<XF16>(1) | (small_int_bits<XF16>(1) << 16);
  const uint4 ones = make_uint4(kOne, kOne, kOne, kOne);
  const floatx4_t zero = {0.f, 0.f, 0.f, 0.f};
  const RegConsts<CD::kNC> dk = CodecOps<CD>::in_registers();  // decoder constants in registers

  float out[TN][MT][MR];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int el = 0; el < MR; ++el) out[t][mt][el] = 0.f;

  // One k-tile of operands: weights and scales of the 4 n-tiles, and the
  // activation fragments of every k-step.
  struct Tile {
    uint4 wv[TN];
    uint32_t sv[TN][4];
    uint4 af[KSTEPS][MT][PARTS];
  };
  auto load_w = [&](int kt, Tile &T) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      T.wv[t] = buf_load16(wrs, wvoff, (kt * 4 + t0 + t) * (kLanes * 16));
      load_scales<BPK * ESZ>(srs, svoff, (kt * kLanes + 16 * (t0 + t)) * (BPK * ESZ), T.sv[t]);
    }
  };
  // Activation fragments of one k-tile.  The main loop covers whole k-tiles
  // with unconditional loads: any branch around a load makes the compiler's
  // wait counting fall back to waiting for every load in flight, prefetch
  // included.  Only the matrix's last k-tile can be partial; it runs after
  // the loop, its missing chunks with zero activations (their codes are
  // zero-padded and their scales and biases zero, so they add nothing).
  auto load_a = [&](int kt, Tile &T) __attribute__((always_inline)) {
    static_for<KSTEPS>([&](auto kc_) {
      constexpr int ks = decltype(kc_)::value;
      constexpr int j = ks / HALVES, h = ks % HALVES;
      const int64_t kp = (int64_t)kt * (KT / 2) + (BITS == 2 ? (32 * j + 8 * g + 4 * h) : (16 * j + 4 * g));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int p = 0; p < PARTS; ++p)
          T.af[ks][mt][p] = *reinterpret_cast<const uint4 *>(arow[mt] + p * a.in_part_stride + kp);
    });
  };
  auto load_a_partial = [&](int kt, Tile &T) __attribute__((always_inline)) {
    const int nch = NC - 4 * kt;  // chunks present in the partial k-tile (1..3)
    static_for<KSTEPS>([&](auto kc_) {
      constexpr int ks = decltype(kc_)::value;
      constexpr int j = ks / HALVES, h = ks % HALVES;
      const int64_t kp = (int64_t)kt * (KT / 2) + (BITS == 2 ? (32 * j + 8 * g + 4 * h) : (16 * j + 4 * g));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int p = 0; p < PARTS; ++p)
          T.af[ks][mt][p] = (j < nch) ? *reinterpret_cast<const uint4 *>(arow[mt] + p * a.in_part_stride + kp)
                                      : make_uint4(0, 0, 0, 0);
    });
  };
  auto compute = [&](int kt, const Tile &T) __attribute__((always_inline)) {
    floatx4_t accW[TN][MT], accC[MT], accX[MT];
    static_for<4>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      {
        uint32_t pr[TN][CD::kPairs];
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const uint32_t wd[4] = {T.wv[t].x, T.wv[t].y, T.wv[t].z, T.wv[t].w};
          CD::extract(wd[j], pr[t], dk);
        }
        static_for<HALVES>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          constexpr int ks = j * HALVES + h;
          constexpr bool first = (j % CPB == 0) && h == 0;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int p = 0; p < PARTS; ++p) {
              const uint4 A = T.af[ks][mt][p];
              const bool fresh = first && p == 0;
              accC[mt] = mfma16<XF16>(A, bc[h], fresh ? zero : accC[mt]);
              if constexpr (AFF) accX[mt] = mfma16<XF16>(A, ones, fresh ? zero : accX[mt]);
#pragma unroll
              for (int t = 0; t < TN; ++t) {
                const uint4 B = make_uint4(pr[t][4 * h], pr[t][4 * h + 1], pr[t][4 * h + 2], pr[t][4 * h + 3]);
                accW[t][mt] = mfma16<XF16>(A, B, fresh ? zero : accW[t][mt]);
              }
            }
          }
        });
        if constexpr (j % CPB == CPB - 1) {
          // block epilogue: out += s (D - C) (+ b X)
          constexpr int bi = j / CPB;
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const uint32_t ent = ESZ == 4 ? T.sv[t][bi] : ((T.sv[t][bi / 2] >> (16 * (bi % 2))) & 0xFFFFu);
            float s = half_to_f32_sel(ent & 0xFFFFu, smask);
            float b = 0.f;
            if constexpr (AFF) b = half_to_f32_sel(ent >> 16, smask);
            if constexpr (CAT) {  // the segment's routing weight scales the block's whole term
              s *= wseg;
              b *= wseg;
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int el = 0; el < MR; ++el) {
                float o = fmaf(s, accW[t][mt][el] - accC[mt][el], out[t][mt][el]);
                if constexpr (AFF) o = fmaf(b, accX[mt][el], o);
                out[t][mt][el] = o;
              }
          }
        }
      }
    });
  };

  // k-tile loop.  PF 0: load and compute one k-tile at a time.  PF 1: the
  // weights and scales of the next k-tile are in flight during the compute;
  // the activations (L2 hits) are issued before that prefetch, so waiting for
  // them never waits for it.  The loop body is straight-line code over two
  // k-tiles (the two register sets swap roles without moves) and the
  // prefetch is unconditional -- past the last whole k-tile it re-reads that
  // tile -- because a load under a branch makes the compiler's wait counting
  // assume the shorter path and wait for the prefetch too.
  // Two row tiles hold twice the activations and accumulators; with a
  // second register set for the prefetch they would spill, so they load
  // one k-tile at a time.
  static_assert(QMOE_GEMV_PREFETCH == 0 || QMOE_GEMV_PREFETCH == 1, "QMOE_GEMV_PREFETCH is 0 or 1");
  constexpr int PF = MT > 1 ? 0 : QMOE_GEMV_PREFETCH;
  Tile TA, TB;
  auto kloop = [&](const int kt0, const int kt1) __attribute__((always_inline)) {
    const int ktf = min(kt1, NC / 4);  // end of this wave's whole k-tiles
    if constexpr (PF == 0) {
      for (int kt = kt0; kt < ktf; ++kt) {
        load_a(kt, TA);
        load_w(kt, TA);
        compute(kt, TA);
      }
    } else if (kt0 < ktf) {
      int kt = kt0;
      if ((ktf - kt0) & 1) {  // odd count: one k-tile without prefetch first
        load_a(kt, TA);
        load_w(kt, TA);
        compute(kt, TA);
        ++kt;
      }
      if (kt < ktf) {
        const int last = ktf - 1;
        load_w(kt, TA);
        // the fences keep the scheduler from starting a k-tile's decode before
        // the loads issued ahead of it, which would wait for the prefetch
        for (; kt < ktf; kt += 2) {
          load_a(kt, TA);
          load_w(kt + 1, TB);
          __builtin_amdgcn_sched_barrier(0);
          compute(kt, TA);
          __builtin_amdgcn_sched_barrier(0);
          load_a(kt + 1, TB);
          load_w(min(kt + 2, last), TA);
          __builtin_amdgcn_sched_barrier(0);
          compute(kt + 1, TB);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // the partial last k-tile of the matrix, when it is this wave's
    for (int kt = max(kt0, ktf); kt < kt1; ++kt) {
      load_a_partial(kt, TA);
      load_w(kt, TA);
      compute(kt, TA);
    }
  };
  // CAT, when every wave's range lies inside one of the k matrices (KS a
  // multiple of k) and holds at most kCatDeep whole k-tiles: all of the
  // wave's weights are requested at once, and the token's h rows (both
  // parts, all k slots) are copied into LDS behind them, so the loop waits for
  // memory once instead of once per k-tile.
  bool deep = false;
  if constexpr (CAT && TN == 1)  // (with 4 n-tiles a wave the requested weights would not fit the registers)
    deep = a.cat_stage && NC % 4 == 0 && KS % a.route_k == 0 && (NKT * a.route_k + KS - 1) / KS <= kCatDeep &&
           a.route_k * 2 * (int)(a.K / 8) <= kCatStagePer * (int)blockDim.x;
  if (CAT && TN == 1 && deep) {
    // the h rows (slot order, no dependence on the routing) are requested
    // first, then the weights once the segment's expert id has arrived
    const int64_t P = a.K / 2;
    const int pieces = (int)(P / 4), total = a.route_k * 2 * pieces;
    u32x4_t hv[kCatStagePer];  // a native vector (a struct array here would stay in scratch memory)
#pragma unroll
    for (int r = 0; r < kCatStagePer; ++r) {
      const int idx = (int)threadIdx.x + r * (int)blockDim.x;
      if (idx < total) {
        const int rp = idx / pieces, pc = idx - rp * pieces;
        hv[r] = *reinterpret_cast<const u32x4_t *>(a.in + (int64_t)(rp >> 1) * a.in_row_pairs +
                                                   (rp & 1) * a.in_part_stride + pc * 4);
      }
    }
    const int jseg = kw0 / NKT, lo = kw0 - jseg * NKT, n = kw1 - kw0;
    const int eseg = __builtin_amdgcn_readfirstlane(cat_e0);
    wrs = code_rsrc(eseg);
    srs = scale_rsrc(eseg);
    wseg = cat_w0;
    Tile W[kCatDeep];
#pragma unroll
    for (int i = 0; i < kCatDeep; ++i) load_w(lo + min(i, n - 1), W[i]);  // past n: the last tile again
    // h of the k slots: [slot][part][K/2 pairs] after the reduction buffer
    uint32_t *sH = reinterpret_cast<uint32_t *>(s_red) + KS * (TN * MT * MR) * kLanes;
#pragma unroll
    for (int r = 0; r < kCatStagePer; ++r) {
      const int idx = (int)threadIdx.x + r * (int)blockDim.x;
      if (idx < total) reinterpret_cast<u32x4_t *>(sH)[idx] = hv[r];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCatDeep; ++i) {
      if (i < n) {
        const int kt = lo + i;
        static_for<KSTEPS>([&](auto kc_) {
          constexpr int ks = decltype(kc_)::value;
          constexpr int jj = ks / HALVES, h = ks % HALVES;
          const int64_t kp = (int64_t)kt * (KT / 2) + (BITS == 2 ? (32 * jj + 8 * g + 4 * h) : (16 * jj + 4 * g));
#pragma unroll
          for (int p = 0; p < PARTS; ++p)
            W[i].af[ks][0][p] = *reinterpret_cast<const uint4 *>(sH + (jseg * 2 + p) * P + kp);
        });
        compute(kt, W[i]);
      }
    }
  } else if constexpr (CAT) {
    // the wave's range over the k matrices: each overlapped matrix j with its
    // expert's weights, the token's h row of slot j and w_j (the first
    // matrix's routing entries were loaded at the start of the kernel)
    for (int j = kw0 / NKT; j < a.route_k && j * NKT < kw1; ++j) {
      const int lo = max(kw0, j * NKT) - j * NKT, hi = min(kw1, (j + 1) * NKT) - j * NKT;
      const bool first = j == kw0 / NKT;
      const int ej = __builtin_amdgcn_readfirstlane(first ? cat_e0 : a.route.ids[j]);
      wrs = code_rsrc(ej);
      srs = scale_rsrc(ej);
      wseg = first ? cat_w0 : a.route.w[j];
      const int64_t prow = j;  // FC1 wrote the one token's h rows in slot order
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) arow[mt] = a.in + prow * a.in_row_pairs;
      kloop(lo, hi);
    }
  } else {
    kloop(kw0, kw1);
  }

  // cross-wave reduction in a fixed order, then the epilogue
  constexpr int NV = TN * MT * MR;  // values per lane
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int el = 0; el < MR; ++el)
        s_red[((wave * TN + t) * MT + mt) * MR * kLanes + el * kLanes + lane] = out[t][mt][el];
  __syncthreads();
  const int64_t N = a.N;
  for (int idx = threadIdx.x; idx < NV * kLanes; idx += blockDim.x) {
    const int lo = idx & (kLanes - 1), q = idx / kLanes;
    const int el = q % MR, mt = (q / MR) % MT, t = q / (MR * MT);
    const int m = 16 * mt + 4 * (lo >> 4) + el;
    const bool valid = m < M;
    float v = 0.f;
    for (int w = 0; w < KS; ++w) v += s_red[w * NV * kLanes + idx];
    const int64_t n = (int64_t)rg * kRowsPerGroup + 16 * (t0 + t) + (lo & 15);
    // EXT instances only: the optional per-expert output bias (FC1 before
    // the activation, FC2 before the routing weight) and the ReLU FFN
    bool relu = false, custom = false;
    if constexpr (EXT && EPI != kEpiStoreAct) {
      if (a.bias) v += half_to_f32_rt(a.bias[(int64_t)e * N + n], a.act_dtype == QMOE_DTYPE_F16);
      relu = a.relu != 0;
      custom = a.sw_custom != 0;
    }
    if constexpr (EPI == kEpiStoreAct) {
      if (valid) a.out_act[(int64_t)m * N + n] = f32_to_act(v, a.act_dtype == QMOE_DTYPE_F16);
    } else if constexpr (SWIGLU) {
      // SwiGLU: rows 2i (gate) and 2i+1 (up) sit in neighbouring lanes;
      // ReLU (EXT, a.relu): every row is one channel, h = max(a, 0)
      const float up = __shfl_xor(v, 1);
      if (valid && (relu || (lo & 1) == 0)) {
        const float gt = v;
        const float h = relu     ? fmaxf(v, 0.f)
                        : custom ? swiglu_cfg(gt, up, a.sw_alpha, a.sw_beta, a.sw_limit)
                                 : gt / (1.f + expf(-gt)) * up;
        const int64_t Ih = relu ? N : N / 2;
        const int64_t i = relu ? n : n / 2;
        int64_t slot_of_row;
        if constexpr (ROUTED) slot_of_row = s_rslot[m];
        else slot_of_row = a.row_list[pbase + m];
        const int64_t p = a.h_by_slot ? slot_of_row : pbase + m;
        const uint16_t hi = f32_to_bf16_rne(h);
        a.h_hi[p * Ih + i] = hi;
        a.h_lo[p * Ih + i] = f32_to_bf16_rne(h - bf16_to_f32(hi));
        if (a.h_dbg) a.h_dbg[slot_of_row * Ih + i] = h;
      }
    } else if constexpr (CAT) {
      if (valid) a.out_act[n] = f32_to_act(v, a.act_dtype == QMOE_DTYPE_F16);  // y of the one token
    } else {
      if (valid) {
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
}

// Kernel of a configuration: rows = the row bound of the launch, tn = 16-row
// tiles per wave (1: four workgroups share a row group's 64 rows), ext = the
// instance with the optional epilogue work (expert bias, ReLU FFN); the
// default instances carry none of it.
template <int QT, bool XF16, int PARTS, int EPI, int MR, int MT, bool EXT>
const void *gemv_ptr_block(int block, int tn) {
  if (tn == 1)
    return block == 64 ? reinterpret_cast<const void *>(&gemv_kernel<QT, XF16, PARTS, EPI, MR, MT, 64, 1, EXT>)
                       : reinterpret_cast<const void *>(&gemv_kernel<QT, XF16, PARTS, EPI, MR, MT, 128, 1, EXT>);
  if (tn != 4) return nullptr;
  return block == 64 ? reinterpret_cast<const void *>(&gemv_kernel<QT, XF16, PARTS, EPI, MR, MT, 64, 4, EXT>)
                     : reinterpret_cast<const void *>(&gemv_kernel<QT, XF16, PARTS, EPI, MR, MT, 128, 4, EXT>);
}

template <int QT, bool XF16, int PARTS, int EPI, bool EXT>
const void *gemv_ptr_rows(int rows, int block, int tn) {
  if (rows <= 1) return gemv_ptr_block<QT, XF16, PARTS, EPI, 1, 1, EXT>(block, tn);
  if constexpr (EPI == kEpiStoreAct) {
    if (rows > 16) return gemv_ptr_block<QT, XF16, PARTS, EPI, 4, 2, EXT>(block, tn);
  }
  return gemv_ptr_block<QT, XF16, PARTS, EPI, 4, 1, EXT>(block, tn);
}

template <int QT, int EPI, bool EXT>
const void *gemv_ptr_fc1(int in_f16, int rows, int block, int tn) {
  // FC1 input: bf16 or f16 rows, or (kGemvInSplitF32) f32 rows given as bf16 hi + lo parts
  return in_f16 == kGemvInSplitF32 ? gemv_ptr_rows<QT, false, 2, EPI, EXT>(rows, block, tn)
         : in_f16                  ? gemv_ptr_rows<QT, true, 1, EPI, EXT>(rows, block, tn)
                                   : gemv_ptr_rows<QT, false, 1, EPI, EXT>(rows, block, tn);
}

template <int QT>
const void *gemv_ptr_qt(int epilogue, int in_f16, int rows, int block, int tn, int ext) {
  if (epilogue == kEpiDown)
    return ext ? gemv_ptr_rows<QT, false, 2, kEpiDown, true>(rows, block, tn)
               : gemv_ptr_rows<QT, false, 2, kEpiDown, false>(rows, block, tn);
  if (epilogue == kEpiDownCat)  // one token, no expert bias
    return (ext || rows > 1) ? nullptr : gemv_ptr_block<QT, false, 2, kEpiDownCat, 1, 1, false>(block, tn);
  if (epilogue == kEpiSwiGLU)
    return ext ? gemv_ptr_fc1<QT, kEpiSwiGLU, true>(in_f16, rows, block, tn)
               : gemv_ptr_fc1<QT, kEpiSwiGLU, false>(in_f16, rows, block, tn);
  if (epilogue == kEpiSwiGLURouted)
    return ext ? gemv_ptr_fc1<QT, kEpiSwiGLURouted, true>(in_f16, rows, block, tn)
               : gemv_ptr_fc1<QT, kEpiSwiGLURouted, false>(in_f16, rows, block, tn);
  return in_f16 ? gemv_ptr_rows<QT, true, 1, kEpiStoreAct, false>(rows, block, tn)
                : gemv_ptr_rows<QT, false, 1, kEpiStoreAct, false>(rows, block, tn);
}

}  // namespace qmoe
