// channels.hip -- gathered-channel expert FFN: only the listed channels of
// each routed expert are read and computed (MoE channel selection explainer:
// top-k channel selection reads the selected channels in full and computes
// them exactly; channels of different experts compete for one per-token
// budget).
//
// A channel c of expert e is the gate row 2c and the up row 2c+1 of FC1 and
// channel c's column of the down projection.  Reading single channels needs
// each of those to be contiguous, so the channel-packed buffer keeps FC1 row
// by row in the canonical byte order and the down projection channel-major
// ([I][H], block scales along H), also row by row.
//
// Two kernels per call; each step is a few dependent memory rounds, so the
// design keeps the rounds few and the loads of a round together:
//
//   chan_fused_kernel   one workgroup of kChanWaves waves per (token, group
//                       of kChanPerWg consecutive list entries).  Round 1:
//                       the wave's list entries, its slice of x and (wave 0)
//                       the token's logits; wave 0 selects the top-k experts
//                       and their weights into LDS.  Round 2: for each of the
//                       wave's kChanEpw entries the gate row (lanes 0-31),
//                       the up row (lanes 32-63) and the down row (all lanes)
//                       with their scales, all issued before any arithmetic.
//                       Then h = silu(g) u from two half-wave dot products
//                       and acc[n] += w_j h D[e][c][n] over the lane's slice
//                       of the H outputs; the waves' sums meet in an LDS
//                       tree in a fixed order and wave 0 writes the group's
//                       partial sums.
//   chan_reduce_kernel  y = the sum of a token's group partial sums in a
//                       fixed order, rounded once to the activation dtype.
//
// Codes are unpacked from canonical bytes with v_cvt_f32_ubyte (field f of
// every byte of a dword masked out, one conversion per weight).  Symmetric
// codes q = u - zp enter FC1 as s (sum u x - zp sum x) per 16-byte piece (one
// scale block) and the down projection as s (u - zp).
#include "codec.hpp"
#include "route_impl.hpp"

namespace qmoe {

constexpr int kChanWaves = 8;                        // waves per chan_fused workgroup
constexpr int kChanEpw = 2;                          // list entries per wave
constexpr int kChanPerWg = kChanWaves * kChanEpw;    // list entries per workgroup
constexpr int kChanReduceWaves = 16;                 // waves per chan_reduce workgroup
static_assert(kChanPerWg == kChanGroupEntries, "group size of the workspace layout");

__device__ inline float ubyte_f(uint32_t w, int b) {
  return (float)((w >> (8 * b)) & 0xFFu);  // v_cvt_f32_ubyte{b}
}

// Loads N consecutive dwords (N = 1, 2, 4 or a multiple of 4; 4N-byte aligned).
template <int N>
__device__ inline void load_dwords(const uint32_t *__restrict__ p, uint32_t (&v)[N]) {
  if constexpr (N == 1) {
    v[0] = p[0];
  } else if constexpr (N == 2) {
    const uint2 q = *reinterpret_cast<const uint2 *>(p);
    v[0] = q.x;
    v[1] = q.y;
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 q = reinterpret_cast<const uint4 *>(p)[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  }
}

// Lane shape for hidden size class HC (H <= 1024 << HC) and field widths
// B1 (FC1) and B2 (down):
//   NPC  16-byte FC1 pieces per lane of a half wave (a row holds H B1 / 128
//        pieces; lane l takes pieces l NPC .. l NPC + NPC - 1);
//   ND   down-row dwords per lane (a row holds H B2 / 32 dwords; lane l takes
//        dwords l ND .. l ND + ND - 1, i.e. ND * 32 / B2 outputs).
template <int B1, int B2, int HC>
struct ChanShape {
  static constexpr int PER1 = 32 / B1, PER2 = 32 / B2;
  static constexpr int NPC = B1 == 4 ? (1 << HC) : (1 << (HC > 0 ? HC - 1 : 0));
  static constexpr int ND = (B2 == 4 ? 2 : 1) << HC;
  static constexpr int NPL = ND * PER2;  // outputs per lane (<= 64, inside one scale block)
};

// FC1 dot products with the matrix cores' decoder: Codec<B1, X16> turns a
// canonical dword (weight i at bits B1 i) into 16-bit float pairs holding
// base_p + u for the weights (p, p + PER1 / 2), exact, and v_dot2 multiplies
// them with the activation pair (x_p, x_{p + PER1/2}) in fp32.  The pairs of
// a dword's activations are built once per piece with v_perm_b32; so is
// cx = sum_p base_p (x_p + x_{p + PER1/2}) + zp sum_i x_i, and a row's piece
// sum is s (dot - cx) = s sum_i (u_i - zp) x_i.
template <bool X16>
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (X16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
  }
}

// A 16-bit float pair (v, v) of a small integer-valued v.
template <bool X16>
__host__ __device__ constexpr uint32_t half_pair(float v) {
  // v = m 2^e with m < 2^8 (all bases + zero points here): bit patterns built
  // from the exponent and mantissa directly
  int e = 0;
  float m = v;
  while (m >= 2.f) {
    m *= 0.5f;
    ++e;
  }
  uint32_t h;
  if (X16) h = (uint32_t)((e + 15) << 10) | (uint32_t)((m - 1.f) * 1024.f);
  else h = (uint32_t)((e + 127) << 7) | (uint32_t)((m - 1.f) * 128.f);
  return h | (h << 16);
}

// Top-k of one token's E <= 64 logits by one wave, in parallel over the
// lanes: lane l's position is the number of logits greater than its own plus
// the number of equal logits of lower index (the selection order of the
// routing kernels), counted against every lane's logit in turn.  The lanes
// of positions j < k write ids[j] and exp(v - max) to LDS; the weights are
// exp(v_j - max) / sum_j exp(v_j - max) with the sum taken in selection
// order, the arithmetic of the routing kernels.
__device__ inline void wave_topk_rank(const float *__restrict__ logits, int E, int k, int32_t *ids, float *w,
                                      float *ex) {
  const int lane = threadIdx.x & 63;
  const float v = lane < E ? logits[lane] : -__builtin_inff();
  int pos = 0;
  for (int m = 0; m < E; ++m) {
    const float vm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), m));
    pos += (vm > v || (vm == v && m < lane)) ? 1 : 0;
  }
  const float vmax = __int_as_float(__builtin_amdgcn_readlane(
      __float_as_int(v), __builtin_ctzll(__ballot(lane < E && pos == 0))));
  const bool sel = lane < E && pos < k;
  const float e = expf(v - vmax);
  if (sel) {
    ids[pos] = lane;
    ex[pos] = e;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += ex[j];
  if (sel) w[pos] = e / sum;
}

// The pairs (base_p, base_p) of a decoder and (1, 1), as compile-time tables.
template <int B, bool X16>
struct BasePairs {
  uint32_t base[Codec<B, X16>::kPairs];
  uint32_t one;
  constexpr BasePairs() : base{}, one(half_pair<X16>(1.f)) {
    for (int p = 0; p < Codec<B, X16>::kPairs; ++p) base[p] = half_pair<X16>(Codec<B, X16>::base(p));
  }
};

template <int B1, int B2, int HC, bool X16>
__global__ __launch_bounds__(kChanWaves * 64) void chan_fused_kernel(ChanArgs a) {
  using SH = ChanShape<B1, B2, HC>;
  using CD = Codec<B1, X16>;
  constexpr int PER1 = SH::PER1, PER2 = SH::PER2, NPC = SH::NPC, ND = SH::ND, NPL = SH::NPL;
  constexpr int NP = CD::kPairs;       // pairs per dword (PER1 / 2)
  constexpr int FPB2 = 8 / B2;
  constexpr uint32_t M2 = B2 == 4 ? 0x0F0F0F0Fu : 0x03030303u;
  constexpr int RS = NPL / 4 + 1;  // float4 per lane in the reduction buffer (one of padding)
  __shared__ TopkScratch s_sc;
  __shared__ int32_t s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ float s_ex[kMaxTopK];
  __shared__ float4 s_red[kChanWaves / 2][64 * RS];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int half = lane >> 5, l = lane & 31;
  const int G = a.groups;
  const int t = blockIdx.x / G, grp = blockIdx.x % G;
  const int per_tok = a.k * a.C;
  const int q0 = grp * kChanPerWg + wv * kChanEpw;
  const int blog1 = a.fc1_block == 128 ? 7 : 6, blog2 = a.dn_block == 128 ? 7 : 6;

  // ---- round 1: list entries, activations, logits (wave 0: top-k)
  int chv = -1;  // lane i < kChanEpw: channel of entry q0 + i
  if (lane < kChanEpw && q0 + lane < per_tok) chv = a.channels[(int64_t)t * per_tok + q0 + lane];
  const int P1 = (int)(a.fc1_row_bytes / 16);  // 16-byte pieces per FC1 row
  const int RD = (int)(a.dn_row_bytes / 4);    // dwords per down row
  uint32_t xr[NPC][2 * PER1];                  // activations of the lane's pieces, two per word
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    const int p = l * NPC + pc;
    if (p < P1) {
      load_dwords<2 * PER1>(reinterpret_cast<const uint32_t *>(a.x + (int64_t)t * a.H + (int64_t)p * 4 * PER1),
                            xr[pc]);
    } else {
#pragma unroll
      for (int i = 0; i < 2 * PER1; ++i) xr[pc][i] = 0u;
    }
  }
  if (wv == 0) {
    if (a.E <= 64) wave_topk_rank(a.logits + (int64_t)t * a.E, a.E, a.k, s_ids, s_w, s_ex);
    else wave_topk<false>(a.logits + (int64_t)t * a.E, a.E, a.k, nullptr, s_w, s_ids, &s_sc);
  }
  __syncthreads();

  // ---- round 2: every row of the wave's entries
  uint32_t c1[kChanEpw][NPC][4];
  uint16_t s1[kChanEpw][NPC];
  uint32_t c2[kChanEpw][ND];
  uint16_t s2[kChanEpw];
  float wj[kChanEpw];
  bool on[kChanEpw];
  const int nb1 = a.H >> blog1, nb2 = a.H >> blog2;
  const uint16_t *sc1 = reinterpret_cast<const uint16_t *>(a.fc1_scales);
  const uint16_t *sc2 = reinterpret_cast<const uint16_t *>(a.dn_scales);
#pragma unroll
  for (int i = 0; i < kChanEpw; ++i) {
    const int c = __builtin_amdgcn_readlane(chv, i);
    on[i] = c >= 0 && c < a.I;  // unused entries read row 0 and add nothing
    const int j = on[i] ? (q0 + i) / a.C : 0;
    const int e = on[i] ? __builtin_amdgcn_readfirstlane(s_ids[j]) : 0;
    wj[i] = on[i] ? s_w[j] : 0.f;
    const int cc = on[i] ? c : 0;
    const int64_t r1 = (int64_t)e * 2 * a.I + 2 * (int64_t)cc + half;
    const uint32_t *row1 = reinterpret_cast<const uint32_t *>(a.fc1 + r1 * a.fc1_row_bytes);
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
      const int p = l * NPC + pc;
      if (p < P1) {
        load_dwords<4>(row1 + 4 * p, c1[i][pc]);
        s1[i][pc] = sc1[r1 * nb1 + ((p * 4 * PER1) >> blog1)];
      } else {
        c1[i][pc][0] = c1[i][pc][1] = c1[i][pc][2] = c1[i][pc][3] = 0u;
        s1[i][pc] = 0;
      }
    }
    const int64_t r2 = (int64_t)e * a.I + cc;
    if (lane * ND < RD) {
      load_dwords<ND>(reinterpret_cast<const uint32_t *>(a.dn + r2 * a.dn_row_bytes) + lane * ND, c2[i]);
      s2[i] = sc2[r2 * nb2 + ((lane * NPL) >> blog2)];
    } else {
#pragma unroll
      for (int d = 0; d < ND; ++d) c2[i][d] = 0u;
      s2[i] = 0;
    }
  }

  // ---- FC1: activation pairs and cx once per piece, then every entry
  const RegConsts<CD::kNC> kc = CodecOps<CD>::in_registers();
  constexpr BasePairs<B1, X16> kb{};
  float dot[kChanEpw];
#pragma unroll
  for (int i = 0; i < kChanEpw; ++i) dot[i] = 0.f;
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    float cb = 0.f, sx = 0.f;  // sum_p base_p (x_p + x_p'), sum of the piece's activations
    float pd[kChanEpw];
#pragma unroll
    for (int i = 0; i < kChanEpw; ++i) pd[i] = 0.f;
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      // dword dw: activations xr[pc][dw NP + m], m < NP, hold (x_2m, x_2m+1);
      // pair p needs (x_p, x_{p+NP})
      const uint32_t *X = &xr[pc][dw * NP];
      uint32_t xp[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p)
        xp[p] = __builtin_amdgcn_perm(X[NP / 2 + p / 2], X[p / 2], (p & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        cb = dot2<X16>(xp[p], kb.base[p], cb);
        sx = dot2<X16>(xp[p], kb.one, sx);
      }
#pragma unroll
      for (int i = 0; i < kChanEpw; ++i) {
        uint32_t wp[NP];
        CD::extract(c1[i][pc][dw], wp, kc);
#pragma unroll
        for (int p = 0; p < NP; ++p) pd[i] = dot2<X16>(wp[p], xp[p], pd[i]);
      }
    }
    const float cx = fmaf((float)a.fc1_zp, sx, cb);
#pragma unroll
    for (int i = 0; i < kChanEpw; ++i) dot[i] = fmaf(half_to_f32_rt(s1[i][pc], a.fc1_sf16), pd[i] - cx, dot[i]);
  }

  // ---- down rows: acc[n] += w_j h_c s u_n; the zero point once at the end
  float acc[NPL];
#pragma unroll
  for (int o = 0; o < NPL; ++o) acc[o] = 0.f;
  float csum = 0.f;
#pragma unroll
  for (int i = 0; i < kChanEpw; ++i) {
    float d1 = dot[i];
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) d1 += __shfl_xor(d1, off);  // within each half wave
    const float g = __shfl(d1, 0), u = __shfl(d1, 32);
    const float coef = on[i] ? wj[i] * (g / (1.f + expf(-g)) * u) : 0.f;
    const float cs = on[i] ? coef * half_to_f32_rt(s2[i], a.dn_sf16) : 0.f;
    csum += cs;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int f = 0; f < FPB2; ++f) {
        const uint32_t v = opaque_v((c2[i][d] >> (B2 * f)) & M2);  // one byte-select conversion per output
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int o = d * PER2 + FPB2 * b + f;  // output lane NPL + o
          acc[o] = fmaf(cs, ubyte_f(v, b), acc[o]);
        }
      }
    }
  }
  const float zc = (float)a.dn_zp * csum;
#pragma unroll
  for (int o = 0; o < NPL; ++o) acc[o] -= zc;

  // ---- the waves' sums: waves w >= 4 store theirs, waves w < 4 add wave
  // w + 4 and store, then each thread adds one float4 of outputs over the
  // four stored sums in order and writes it (a fixed order throughout)
  static_assert(kChanWaves == 8, "two-level reduction over 8 waves");
  if (wv >= 4) {
#pragma unroll
    for (int o = 0; o < NPL / 4; ++o)
      s_red[wv - 4][lane * RS + o] = make_float4(acc[4 * o], acc[4 * o + 1], acc[4 * o + 2], acc[4 * o + 3]);
  }
  __syncthreads();
  if (wv < 4) {
#pragma unroll
    for (int o = 0; o < NPL / 4; ++o) {
      float4 r = s_red[wv][lane * RS + o];
      r.x += acc[4 * o];
      r.y += acc[4 * o + 1];
      r.z += acc[4 * o + 2];
      r.w += acc[4 * o + 3];
      s_red[wv][lane * RS + o] = r;
    }
  }
  __syncthreads();
  float *dst = a.partial + ((int64_t)t * G + grp) * a.H;
  const int nvec = (a.H + 3) / 4;  // float4 outputs (lane L holds outputs L NPL .. L NPL + NPL - 1)
  for (int idx = threadIdx.x; idx < 64 * (NPL / 4); idx += kChanWaves * 64) {
    const int L = idx / (NPL / 4), o = idx % (NPL / 4);
    const int n4 = L * (NPL / 4) + o;
    if (n4 < nvec) {
      float4 r = s_red[0][L * RS + o];
#pragma unroll
      for (int w = 1; w < kChanWaves / 2; ++w) {
        const float4 q = s_red[w][L * RS + o];
        r.x += q.x;
        r.y += q.y;
        r.z += q.z;
        r.w += q.w;
      }
      reinterpret_cast<float4 *>(dst)[n4] = r;
    }
  }
}

// ------------------------------------------------------------ base-3 rows
// Both matrices TERNARY_B3: every row is a run of block records (the digit
// bytes of B weights, five per byte, then the block's 16-bit scale in the
// record's last two bytes; RW = record bytes / 4 dwords).  A "unit" is one
// record dword: its (up to) four digit bytes hold 20 consecutive weights,
// b B + 20 j + i for record b, dword j, i < min(20, B - 20 j); the last
// dword's other bytes are padding and the scale, whose digits are masked.
// A 256-entry table in LDS turns a byte into its five base-3 digits (least
// significant first) as bytes, read with v_cvt_f32_ubyte.
__device__ inline void b3_table(uint2 *lut) {
  for (int v = threadIdx.x; v < 256; v += blockDim.x) {
    uint32_t d[5] = {0u, 0u, 0u, 0u, 0u};
    if (v < 243) {
      int r = v;
      for (int i = 0; i < 5; ++i) {
        d[i] = (uint32_t)(r % 3);
        r /= 3;
      }
    }
    lut[v] = make_uint2(d[0] | (d[1] << 8) | (d[2] << 16) | (d[3] << 24), d[4]);
  }
}

// The 20 digits of a unit dword as floats.
__device__ inline void b3_digits(const uint2 *lut, uint32_t w, float (&dg)[20]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint2 e = lut[(w >> (8 * m)) & 0xFFu];
#pragma unroll
    for (int i = 0; i < 4; ++i) dg[5 * m + i] = ubyte_f(e.x, i);
    dg[5 * m + 4] = ubyte_f(e.y, 0);
  }
}

// The same workgroup shape and steps as chan_fused_kernel; HC: H <= 1024 << HC.
template <int HC>
__global__ __launch_bounds__(kChanWaves * 64) void chan_b3_kernel(ChanArgs a) {
  constexpr int NU1 = 2 << HC;   // units per lane of a half wave (FC1 rows: <= 64 << HC units)
  constexpr int NU2 = 1 << HC;   // units per lane (down rows)
  constexpr int NPL = 20 * NU2;  // down outputs per lane
  constexpr int RS = NPL / 4 + 1;
  __shared__ TopkScratch s_sc;
  __shared__ int32_t s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ float s_ex[kMaxTopK];
  __shared__ uint2 s_lut[256];
  __shared__ __align__(16) float s_x[(1024 << HC) + 32];
  __shared__ float4 s_red[kChanWaves / 2][64 * RS];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int half = lane >> 5, l = lane & 31;
  const int G = a.groups;
  const int t = blockIdx.x / G, grp = blockIdx.x % G;
  const int per_tok = a.k * a.C;
  const int q0 = grp * kChanPerWg + wv * kChanEpw;
  const int RW1 = b3_record_bytes(a.fc1_block) / 4, RW2 = b3_record_bytes(a.dn_block) / 4;
  const int U1 = (a.H / a.fc1_block) * RW1, U2 = (a.H / a.dn_block) * RW2;

  // ---- round 1: list entries, activations (to LDS), logits; digit table
  int chv = -1;
  if (lane < kChanEpw && q0 + lane < per_tok) chv = a.channels[(int64_t)t * per_tok + q0 + lane];
  for (int n = threadIdx.x; n < a.H + 32; n += blockDim.x)
    s_x[n] = n < a.H ? half_to_f32_rt(a.x[(int64_t)t * a.H + n], a.x_f16) : 0.f;
  b3_table(s_lut);
  if (wv == 0) {
    if (a.E <= 64) wave_topk_rank(a.logits + (int64_t)t * a.E, a.E, a.k, s_ids, s_w, s_ex);
    else wave_topk<false>(a.logits + (int64_t)t * a.E, a.E, a.k, nullptr, s_w, s_ids, &s_sc);
  }
  __syncthreads();

  // ---- round 2: every unit dword and its record's scale dword, all entries
  uint32_t c1[kChanEpw][NU1], k1[kChanEpw][NU1];
  uint32_t c2[kChanEpw][NU2], k2[kChanEpw][NU2];
  float wj[kChanEpw];
  bool on[kChanEpw];
#pragma unroll
  for (int i = 0; i < kChanEpw; ++i) {
    const int c = __builtin_amdgcn_readlane(chv, i);
    on[i] = c >= 0 && c < a.I;
    const int j = on[i] ? (q0 + i) / a.C : 0;
    const int e = on[i] ? __builtin_amdgcn_readfirstlane(s_ids[j]) : 0;
    wj[i] = on[i] ? s_w[j] : 0.f;
    const int cc = on[i] ? c : 0;
    const uint32_t *row1 = reinterpret_cast<const uint32_t *>(
        a.fc1 + ((int64_t)e * 2 * a.I + 2 * (int64_t)cc + half) * a.fc1_row_bytes);
#pragma unroll
    for (int iu = 0; iu < NU1; ++iu) {
      const int u = l + 32 * iu;
      const int uc = u < U1 ? u : U1 - 1;
      c1[i][iu] = row1[uc];
      k1[i][iu] = row1[(uc / RW1) * RW1 + RW1 - 1];
    }
    const uint32_t *row2 =
        reinterpret_cast<const uint32_t *>(a.dn + ((int64_t)e * a.I + cc) * a.dn_row_bytes);
#pragma unroll
    for (int iu = 0; iu < NU2; ++iu) {
      const int u = lane + 64 * iu;
      const int uc = u < U2 ? u : U2 - 1;
      c2[i][iu] = row2[uc];
      k2[i][iu] = row2[(uc / RW2) * RW2 + RW2 - 1];
    }
  }

  // ---- FC1: per unit, su = sum d x and sx = sum x over its weights
  float dot[kChanEpw];
#pragma unroll
  for (int i = 0; i < kChanEpw; ++i) dot[i] = 0.f;
#pragma unroll
  for (int iu = 0; iu < NU1; ++iu) {
    const int u = l + 32 * iu;
    const int b = u / RW1, jd = u - b * RW1;
    const int cnt = u < U1 ? min(20, a.fc1_block - 20 * jd) : 0;
    const int base = b * a.fc1_block + 20 * jd;
    float xv[20];
    float sx = 0.f;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const float4 v = u < U1 ? *reinterpret_cast<const float4 *>(&s_x[base + 4 * q]) : make_float4(0.f, 0.f, 0.f, 0.f);
      xv[4 * q] = v.x;
      xv[4 * q + 1] = v.y;
      xv[4 * q + 2] = v.z;
      xv[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int m = 0; m < 20; ++m) {
      xv[m] = m < cnt ? xv[m] : 0.f;
      sx += xv[m];
    }
#pragma unroll
    for (int i = 0; i < kChanEpw; ++i) {
      float dg[20];
      b3_digits(s_lut, c1[i][iu], dg);
      float su = 0.f;
#pragma unroll
      for (int m = 0; m < 20; ++m) su = fmaf(dg[m], xv[m], su);
      const float sc = half_to_f32_rt(k1[i][iu] >> 16, a.fc1_sf16);
      dot[i] = fmaf(sc, su - sx, dot[i]);  // q = digit - 1
    }
  }

  // ---- down rows: acc += w_j h_c s d per unit; the zero point per unit at the end
  float acc[NPL];
#pragma unroll
  for (int o = 0; o < NPL; ++o) acc[o] = 0.f;
  float csum[NU2];
#pragma unroll
  for (int iu = 0; iu < NU2; ++iu) csum[iu] = 0.f;
#pragma unroll
  for (int i = 0; i < kChanEpw; ++i) {
    float d1 = dot[i];
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) d1 += __shfl_xor(d1, off);
    const float g = __shfl(d1, 0), uu = __shfl(d1, 32);
    const float coef = on[i] ? wj[i] * (g / (1.f + expf(-g)) * uu) : 0.f;
#pragma unroll
    for (int iu = 0; iu < NU2; ++iu) {
      const float cs = on[i] ? coef * half_to_f32_rt(k2[i][iu] >> 16, a.dn_sf16) : 0.f;
      csum[iu] += cs;
      float dg[20];
      b3_digits(s_lut, c2[i][iu], dg);
#pragma unroll
      for (int m = 0; m < 20; ++m) acc[20 * iu + m] = fmaf(cs, dg[m], acc[20 * iu + m]);
    }
  }
#pragma unroll
  for (int iu = 0; iu < NU2; ++iu)
#pragma unroll
    for (int m = 0; m < 20; ++m) acc[20 * iu + m] -= csum[iu];  // zero point 1

  // ---- the waves' sums (fixed order, as in chan_fused_kernel), then the
  // valid outputs of each unit
  if (wv >= 4) {
#pragma unroll
    for (int o = 0; o < NPL / 4; ++o)
      s_red[wv - 4][lane * RS + o] = make_float4(acc[4 * o], acc[4 * o + 1], acc[4 * o + 2], acc[4 * o + 3]);
  }
  __syncthreads();
  if (wv < 4) {
#pragma unroll
    for (int o = 0; o < NPL / 4; ++o) {
      float4 r = s_red[wv][lane * RS + o];
      r.x += acc[4 * o];
      r.y += acc[4 * o + 1];
      r.z += acc[4 * o + 2];
      r.w += acc[4 * o + 3];
      s_red[wv][lane * RS + o] = r;
    }
  }
  __syncthreads();
  float *dst = a.partial + ((int64_t)t * G + grp) * a.H;
  for (int idx = threadIdx.x; idx < 64 * (NPL / 4); idx += kChanWaves * 64) {
    const int L = idx / (NPL / 4), o = idx % (NPL / 4);
    const int u = L + 64 * (o / 5);
    if (u >= U2) continue;
    const int b = u / RW2, jd = u - b * RW2;
    const int cnt = min(20, a.dn_block - 20 * jd);
    float4 r = s_red[0][L * RS + o];
#pragma unroll
    for (int w = 1; w < kChanWaves / 2; ++w) {
      const float4 q = s_red[w][L * RS + o];
      r.x += q.x;
      r.y += q.y;
      r.z += q.z;
      r.w += q.w;
    }
    const int m0 = 4 * (o % 5);
    const int64_t n0 = (int64_t)b * a.dn_block + 20 * jd + m0;
    const float rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (m0 + m < cnt) dst[n0 + m] = rv[m];
  }
}

// One thread per (row, block): a canonical base-3 block (ceil(B/5) bytes) and
// its scale into one record; bytes holding more digits than they may are
// counted.
__global__ __launch_bounds__(256) void pack_b3_kernel(const uint8_t *__restrict__ codes,
                                                      const uint16_t *__restrict__ scales, int64_t rows, int nblk,
                                                      int block, uint8_t *__restrict__ dst, uint32_t *count) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= rows * nblk) return;
  const int per = b3_block_bytes(block), R = b3_record_bytes(block);
  const int last = block % 5 ? block % 5 : 5;  // digits of the block's last byte
  const uint8_t *src = codes + id * per;       // rows are nblk blocks of per bytes, back to back
  uint32_t *out = reinterpret_cast<uint32_t *>(dst + id * R);
  uint32_t bad = 0;
  for (int wd = 0; wd < R / 4; ++wd) {
    uint32_t w = 0;
    for (int m = 0; m < 4; ++m) {
      const int j = 4 * wd + m;
      uint32_t v = 0;
      if (j < per) {
        v = src[j];
        const uint32_t limit = j == per - 1 ? (last == 5 ? 243u : (last == 4 ? 81u : last == 3 ? 27u : last == 2 ? 9u : 3u))
                                            : 243u;
        bad += v >= limit ? 1u : 0u;
      } else if (j >= R - 2) {
        v = (scales[id] >> (8 * (j - (R - 2)))) & 0xFFu;
      }
      w |= v << (8 * m);
    }
    out[wd] = w;
  }
  if (bad) atomicAdd(count, bad);
}

hipError_t launch_pack_b3_records(const uint8_t *codes, const uint16_t *scales, int64_t rows, int64_t K, int block,
                                  uint8_t *dst, uint32_t *count, hipStream_t s) {
  const int nblk = (int)(K / block);
  const int64_t n = rows * nblk;
  if (n == 0) return hipSuccess;
  return qlaunch(pack_b3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, scales, rows, nblk, block,
                 dst, count);
}

// Workgroup (t, 64 outputs): wave v sums groups v, v + kChanReduceWaves, ...
// in order, then wave 0 adds the waves' sums in wave order.
__global__ __launch_bounds__(kChanReduceWaves * 64) void chan_reduce_kernel(ChanArgs a) {
  __shared__ float part[kChanReduceWaves][64];
  const int lane = threadIdx.x & 63, v = threadIdx.x >> 6;
  const int nchunk = (a.H + 63) / 64;
  const int t = blockIdx.x / nchunk, n = (blockIdx.x % nchunk) * 64 + lane;
  float s = 0.f;
  if (n < a.H) {
    const float *p = a.partial + (int64_t)t * a.groups * a.H + n;
#pragma unroll 8
    for (int g = v; g < a.groups; g += kChanReduceWaves) s += p[(int64_t)g * a.H];
  }
  part[v][lane] = s;
  __syncthreads();
  if (v == 0 && n < a.H) {
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kChanReduceWaves; ++w) y += part[w][lane];
    a.y[(int64_t)t * a.H + n] = f32_to_act(y, a.x_f16);
  }
}

// Counts 2-bit fields equal to 3 (the invalid ternary value).
__global__ __launch_bounds__(256) void count_ternary3_kernel(const uint32_t *p, int64_t ndw, uint32_t *count) {
  uint32_t c = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ndw; i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t w = p[i];
    c += __popc(w & (w >> 1) & 0x55555555u);
  }
  if (c) atomicAdd(count, c);
}

hipError_t launch_count_invalid_ternary(const uint8_t *p, int64_t bytes, uint32_t *count, hipStream_t s) {
  const int64_t ndw = bytes / 4;
  if (ndw == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((ndw + 255) / 256, 4096);
  return qlaunch(count_ternary3_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                 reinterpret_cast<const uint32_t *>(p), ndw, count);
}

template <int B1, int B2, bool X16>
hipError_t launch_fused_bits(const ChanArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.T * a.groups)), block(kChanWaves * 64);
  if (a.H <= 1024) return qlaunch(chan_fused_kernel<B1, B2, 0, X16>, grid, block, 0, s, a);
  if (a.H <= 2048) return qlaunch(chan_fused_kernel<B1, B2, 1, X16>, grid, block, 0, s, a);
  return qlaunch(chan_fused_kernel<B1, B2, 2, X16>, grid, block, 0, s, a);
}

template <bool X16>
hipError_t launch_fused(const ChanArgs &a, hipStream_t s) {
  if (a.fc1_bits == 4)
    return a.dn_bits == 4 ? launch_fused_bits<4, 4, X16>(a, s) : launch_fused_bits<4, 2, X16>(a, s);
  return a.dn_bits == 4 ? launch_fused_bits<2, 4, X16>(a, s) : launch_fused_bits<2, 2, X16>(a, s);
}

hipError_t launch_channels(const ChanArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.H > kChanMaxHidden) return hipErrorInvalidValue;
  hipError_t e;
  if (a.b3) {
    const dim3 grid((unsigned)((int64_t)a.T * a.groups)), block(kChanWaves * 64);
    if (a.H > kChanMaxHiddenB3) return hipErrorInvalidValue;
    e = a.H <= 1024 ? qlaunch(chan_b3_kernel<0>, grid, block, 0, s, a) : qlaunch(chan_b3_kernel<1>, grid, block, 0, s, a);
  } else {
    e = a.x_f16 ? launch_fused<true>(a, s) : launch_fused<false>(a, s);
  }
  if (e != hipSuccess) return e;
  const int64_t blocks = (int64_t)a.T * ((a.H + 63) / 64);
  return qlaunch(chan_reduce_kernel, dim3((unsigned)blocks), dim3(kChanReduceWaves * 64), 0, s, a);
}

}  // namespace qmoe
