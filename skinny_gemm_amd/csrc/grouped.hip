// grouped.hip -- grouped larger-M path: tiles of 64 routed rows x 128 or 256 outputs
// per workgroup, MFMA (v_mfma_f32_16x16x32_f16) on weights dequantized once
// per tile in registers.
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
#include <float.h>

#include "codec.hpp"
#include "gemv_impl.hpp"
#include "qmoe_internal.h"

namespace qmoe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Power of two p with amax * p < 2^lim (1 for amax = 0 or non-finite).
__device__ inline float pow2_below(float amax, int lim) {
  if (!(amax > 0.f) || !(amax <= FLT_MAX)) return 1.f;
  int e;
  frexpf(amax, &e);  // amax < 2^e
  int s = lim - e;
  s = max(-120, min(120, s));
  return ldexpf(1.f, s);
}

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

// ---------------------------------------------------------------- GEMM
constexpr int kMaxAffineBlocks = kGroupedMaxAffineBlocks;

// Input modes: 16-bit rows (bf16 or f16) scaled while staged, fp32 rows
// split into f16 hi + lo while staged, or f16 rows already scaled (copied).
enum { kInBf16 = 0, kInF16 = 1, kInF32 = 2, kInScaled = 3 };

template <int QT, int EPI, int INM>
__global__ __launch_bounds__(256) void grouped_kernel(const GroupedArgs a) {
  constexpr bool IN_F32 = INM == kInF32, IN_F16 = INM == kInF16, PRE = INM == kInScaled;
  using TR = QtTraits<QT>;
  using CD = Codec<TR::kBits, true>;
  constexpr int KC = 128 / TR::kBits;  // k per 16-B chunk: 32 (4-bit) or 64 (2-bit)
  constexpr int NPART = IN_F32 ? 2 : 1;  // fp32 input: f16 hi + lo parts (about 22 bits)
  constexpr int KT = IN_F32 ? 64 : 128;  // k per staged tile (two buffers of NPART parts fit the LDS)
  constexpr int CPT = KT / KC;         // chunks per tile
  constexpr int KS = KT / 32;          // MFMA k-steps per tile
  constexpr int APAD = 8;              // row padding of the staged tile (halves)
  constexpr bool AFF = TR::kAffine;
  // codes enter the MFMA as q = u - zc: the symmetric codes, and affine codes
  // recentred to [-2^(b-1), 2^(b-1)-1] (bias b + zc*s added in the epilogue)
  constexpr int ZC = AFF ? (1 << (TR::kBits - 1)) : TR::kZeroPoint;
  // codes of more than one significant bit times an 11-bit (f16) scale do not
  // fit f16: the scale is split into an 8-bit head and its tail (two MFMAs)
  constexpr bool MULTIBIT = (QT == QMOE_QTYPE_SYM_INT4 || QT == QMOE_QTYPE_AFFINE_INT4);

  __shared__ _Float16 sA[2][NPART][kTileM][KT + APAD];
  __shared__ int s_row[kTileM];
  __shared__ float s_rsc[kTileM];
  __shared__ float s_X[AFF ? kTileM : 1][AFF ? kMaxAffineBlocks : 1];  // per-row block sums of x

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // 16-column slices per wave: 4 (tile of 256 outputs) for the fp32 FC2
  // input, whose f16 hi + lo parts double the MFMAs per dequantized weight
  // fragment; 2 (128 outputs) for 16-bit inputs, where the occupancy of the
  // narrower tile measured faster
  constexpr int NJ = IN_F32 ? 4 : 2;
  constexpr int TW = 4 * 16 * NJ;  // outputs per tile
  const int ntn = (int)((a.N + TW - 1) / TW);

  // XCD-aware remap: blocks are dealt round-robin to 8 XCDs; give each XCD a
  // contiguous range of tiles (n-tile major, row tiles of an expert adjacent)
  const int G = gridDim.x;
  const int bid = (G % 8 == 0) ? ((int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8)) : (int)blockIdx.x;
  const int tiles_m = G / ntn;
  const int nt = bid / tiles_m, tile = bid - nt * tiles_m;

  int e, p0, rows;
  if (a.dense_M > 0) {
    e = 0;
    p0 = tile * kTileM;
    rows = min(kTileM, a.dense_M - p0);
  } else {
    const int4 ti = a.tile_info[tile];
    e = ti.x;
    p0 = ti.y;
    rows = ti.z;
  }
  if (rows <= 0) return;

  if (threadIdx.x < kTileM) {
    const int r = threadIdx.x;
    int inrow = -1;
    float sc = 0.f;
    if (r < rows) {
      const int p = p0 + r;
      inrow = (a.dense_M > 0) ? p : (a.in_gather_token ? a.token_of[p] : p);
      sc = IN_F32 ? pow2_below(__uint_as_float(a.in_rowmax[inrow]), 14) : a.in_rowsc[inrow];
    }
    s_row[r] = inrow;
    s_rsc[r] = sc;
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
  const bool split = MULTIBIT && sf16;

  floatx4_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // staging assignment: 4 threads per row, KT/4 consecutive k each
  constexpr int SEG = KT / 4;
  const int st_r = threadIdx.x >> 2, st_k = (threadIdx.x & 3) * SEG;
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
  auto load_b = [&](int64_t kt, uint32_t (&bw)[CPT][NJ], uint32_t (&sv)[CPT][NJ]) __attribute__((always_inline)) {
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
        sv[c][j] = AFF ? __builtin_amdgcn_raw_buffer_load_b32(srs, svo, sj, 0)
                       : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(srs, svo, sj, 0);
      }
    });
  };
  const RegConsts<CD::kNC> dk = CodecOps<CD>::in_registers();  // decoder constants in registers
  auto compute = [&](int buf, const uint32_t (&bw)[CPT][NJ], const uint32_t (&sv)[CPT][NJ])
                     __attribute__((always_inline)) {
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
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int pp = 0; pp < NPART; ++pp) {
          const half8_t af = *reinterpret_cast<const half8_t *>(&sA[buf][pp][16 * i + (lane & 15)][koff]);
          if (wave_on) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
              if (split) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bl[j], acc[i][j], 0, 0, 0);
            }
          }
        }
      }
    });
  };

  // Two-stage pipeline over the k-tiles: the next tile's weights, scales and
  // activations are loaded while the current one is multiplied; one barrier
  // per tile (the staged buffers alternate).
  uint32_t bwA[CPT][NJ], svA[CPT][NJ], bwB[CPT][NJ], svB[CPT][NJ];
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
    }
    compute(buf, bwA, svA);
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
        for (int i = 0; i < 4; ++i)
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
    bv[j] = a.bias ? half_to_f32_rt(a.bias[(int64_t)e * a.N + nw + 16 * j + (lane & 15)],
                                    a.act_dtype == QMOE_DTYPE_F16)
                   : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int el = 0; el < 4; ++el) {
      const int m = 16 * i + 4 * g + el;
      const bool valid = m < rows && wave_on;
      const float inv = valid ? winv / s_rsc[m] : 0.f;
      float hmax = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float v = fmaf(acc[i][j][el], inv, bv[j]);
        const int64_t n = nw + 16 * j + (lane & 15);
        if constexpr (EPI == kGEpiSwiGLU) {
          // SwiGLU over neighbouring gate/up lanes, or (a.relu) h = max(a, 0) per row
          const float up = __shfl_xor(v, 1);
          if (valid && (a.relu || (lane & 1) == 0)) {
            const float h = a.relu ? fmaxf(v, 0.f) : v / (1.f + expf(-v)) * up;
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
}

template <int QT, int EPI>
hipError_t launch_grouped_in(const GroupedArgs &a, int grid, hipStream_t s) {
  if (a.in_f32) return qlaunch(grouped_kernel<QT, EPI, kInF32>, dim3(grid), dim3(256), 0, s, a);
  if (a.in_scaled) return qlaunch(grouped_kernel<QT, EPI, kInScaled>, dim3(grid), dim3(256), 0, s, a);
  if (a.in_f16) return qlaunch(grouped_kernel<QT, EPI, kInF16>, dim3(grid), dim3(256), 0, s, a);
  return qlaunch(grouped_kernel<QT, EPI, kInBf16>, dim3(grid), dim3(256), 0, s, a);
}

template <int QT>
hipError_t launch_grouped_qt(const GroupedArgs &a, int epi, int grid, hipStream_t s) {
  if (epi == kGEpiSwiGLU) return launch_grouped_in<QT, kGEpiSwiGLU>(a, grid, s);
  if (epi == kGEpiStoreF32) return launch_grouped_in<QT, kGEpiStoreF32>(a, grid, s);
  return launch_grouped_in<QT, kGEpiStoreAct>(a, grid, s);
}

hipError_t launch_grouped(const GroupedArgs &a, int epilogue, int grid_tiles, hipStream_t s) {
  const int tw = a.in_f32 ? kTileNWide : kTileN;  // as the kernel's tile width
  const int ntn = (int)((a.N + tw - 1) / tw);
  const int grid = grid_tiles * ntn;
  if (grid == 0) return hipSuccess;
  switch (a.qtype) {
    case QMOE_QTYPE_SYM_INT4: return launch_grouped_qt<QMOE_QTYPE_SYM_INT4>(a, epilogue, grid, s);
    case QMOE_QTYPE_SYM_INT2: return launch_grouped_qt<QMOE_QTYPE_SYM_INT2>(a, epilogue, grid, s);
    case QMOE_QTYPE_TERNARY: return launch_grouped_qt<QMOE_QTYPE_TERNARY>(a, epilogue, grid, s);
    case QMOE_QTYPE_AFFINE_INT2: return launch_grouped_qt<QMOE_QTYPE_AFFINE_INT2>(a, epilogue, grid, s);
    default: return launch_grouped_qt<QMOE_QTYPE_AFFINE_INT4>(a, epilogue, grid, s);
  }
}

hipError_t launch_rowscale(const void *x, int rows, int64_t K, int in_f16, float *rowsc, uint16_t *xs,
                           hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return qlaunch(rowscale_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, (const uint16_t *)x, rows, K, in_f16,
                 rowsc, xs);
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
