// qmoe_internal.h -- layout arithmetic and launch argument blocks shared by
// the host ABI (abi.hip) and the gfx950 kernels.  Host + device.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "../../include/qmoe.h"

namespace qmoe {

constexpr int kLanes = 64;            // wavefront width on CDNA4
constexpr int kRowsPerGroup = 64;     // one output row per lane in the GEMV layout
constexpr int kChunkBytes = 16;       // one 128-bit load per lane
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;
constexpr int kGemvMaxRows = 16;      // rows per expert on the GEMV path (one MFMA row tile)
constexpr int64_t kAlign = 256;

__host__ __device__ inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

__host__ __device__ inline int qtype_bits(int qt) {
  return (qt == QMOE_QTYPE_SYM_INT4 || qt == QMOE_QTYPE_AFFINE_INT4) ? 4 : 2;
}
// Base-3 ternary rows: ceil(B/5) digit bytes per block of B weights in the
// canonical form; in the channel-packed buffer one 4-byte aligned record of
// the digit bytes and the block's 16-bit scale in its last two bytes.
__host__ __device__ inline int b3_block_bytes(int block) { return (block + 4) / 5; }
__host__ __device__ inline int b3_record_bytes(int block) { return (b3_block_bytes(block) + 2 + 3) / 4 * 4; }
__host__ __device__ inline bool qtype_affine(int qt) {
  return qt == QMOE_QTYPE_AFFINE_INT2 || qt == QMOE_QTYPE_AFFINE_INT4;
}
// Zero point folded into the symmetric codes: q = u - zp.
__host__ __device__ inline int qtype_zero_point(int qt) {
  switch (qt) {
    case QMOE_QTYPE_SYM_INT4: return 8;
    case QMOE_QTYPE_SYM_INT2: return 2;
    case QMOE_QTYPE_TERNARY: return 1;
    case QMOE_QTYPE_TERNARY_B3: return 1;
    default: return 0;
  }
}

// Prepacked layout of one quantized matrix W [N][K] (one expert).
//
// A chunk is 16 B of one row: kc = 128/bits consecutive weights.  Inside a
// chunk, dword d covers weights [d*wpd, (d+1)*wpd) (wpd = 32/bits) and weight
// pair j = (2j, 2j+1) of the dword keeps its even weight in the low half-word
// and its odd weight in the high half-word at the same bit offset (4j for
// 4-bit, 2j for 2-bit), so one AND-OR places a pair into the mantissas of two
// 16-bit floats.
//
// codes : [N/64 row groups][NKT k-tiles][4 n-tiles][64 lanes][16 B].  A
//         k-tile is 4 chunks (kt = 4*kc weights).  Lane r + 16 g of n-tile t
//         holds, as its dword j, dword g of chunk j of row 64 rg + 16 t + r:
//         one 1 KiB contiguous wave load gives every lane the MFMA B operand
//         of row (lane % 16) for k-group (lane / 16) of four chunks, and one
//         chunk is one block-aligned group of MFMA k-steps.  A partial last
//         k-tile is padded with zero chunks.
// scales: [N/64][NKT][64 rows][bpk blocks] x (scale) or (scale | bias << 16),
//         bpk = kt / block blocks per k-tile (padded entries are zero): the
//         lanes of row r read all scales of a k-tile with one load.
struct MatLayout {
  int qtype, bits, block, sdtype;
  bool affine;
  int64_t N, K;
  int64_t RG;    // row groups
  int kc;        // weights per lane chunk (16 B)
  int64_t NC;    // chunks per row
  int64_t NKT;   // k-tiles per row (4 chunks each)
  int64_t nblk;  // blocks per row
  int cpb;       // chunks per block
  int bpk;       // blocks per k-tile
  int scale_elem;         // bytes per block entry (2 or 4)
  int64_t codes_bytes;
  int64_t scales_off;     // from the start of the expert's matrix
  int64_t scales_bytes;
  int64_t stride;         // bytes per expert

  __host__ __device__ static MatLayout make(const qmoe_qmatrix_desc &d) {
    MatLayout L{};
    L.qtype = d.qtype;
    L.bits = qtype_bits(d.qtype);
    L.block = d.block;
    L.sdtype = d.scale_dtype;
    L.affine = qtype_affine(d.qtype);
    L.N = d.rows;
    L.K = d.cols;
    L.RG = d.rows / kRowsPerGroup;
    L.kc = kChunkBytes * 8 / L.bits;
    L.NC = d.cols / L.kc;
    L.NKT = (L.NC + 3) / 4;
    L.nblk = d.cols / d.block;
    L.cpb = d.block / L.kc;
    L.bpk = 4 * L.kc / d.block;
    L.scale_elem = L.affine ? 4 : 2;
    L.codes_bytes = L.RG * L.NKT * 4 * kLanes * kChunkBytes;
    L.scales_off = align_up(L.codes_bytes, kAlign);
    L.scales_bytes = L.RG * L.NKT * kLanes * L.bpk * L.scale_elem;
    L.stride = L.scales_off + align_up(L.scales_bytes, kAlign);
    return L;
  }
  // Byte offset (from the expert's matrix) of the 4-byte word holding
  // dword `d` of chunk `c` of row `n`.
  __host__ __device__ int64_t code_word_offset(int64_t n, int64_t c, int d) const {
    const int64_t rg = n / kRowsPerGroup, t = (n % kRowsPerGroup) / 16, r = n % 16;
    const int64_t kt = c / 4, j = c % 4;
    return ((((rg * NKT + kt) * 4 + t) * kLanes + r + 16 * d) * kChunkBytes) + 4 * j;
  }
  // Index (in entries of scale_elem bytes) of the scale of row n, block b.
  __host__ __device__ int64_t scale_index(int64_t n, int64_t b) const {
    const int64_t rg = n / kRowsPerGroup, rl = n % kRowsPerGroup;
    return ((rg * NKT + b / bpk) * kLanes + rl) * bpk + b % bpk;
  }
};

// Prepacked MoE buffer: [header 256 B][FC1: E x stride1][FC2: E x stride2].
constexpr int64_t kHeaderBytes = 256;
constexpr uint64_t kPackMagic = 0x31304b50454f4d51ull;  // "QMOEPK01"
constexpr int64_t kErrWordOff = 128;                     // u32 invalid-field counter

// wsc_off: float [2][E] power-of-two pre-scales of the MFMA path (FC1, FC2).
struct MoeLayout {
  MatLayout fc1, fc2;
  int64_t fc1_off, fc2_off, wsc_off, total;
  static MoeLayout make(const qmoe_layer_desc &d) {
    MoeLayout L{};
    L.fc1 = MatLayout::make(d.fc1);
    L.fc2 = MatLayout::make(d.fc2);
    L.fc1_off = kHeaderBytes;
    L.fc2_off = L.fc1_off + (int64_t)d.num_experts * L.fc1.stride;
    L.wsc_off = L.fc2_off + (int64_t)d.num_experts * L.fc2.stride;
    L.total = L.wsc_off + align_up(2 * (int64_t)d.num_experts * 4, kAlign);
    return L;
  }
};

// Dense (linear) prepacked buffer: [matrix][tail 256 B: u32 error word at +0,
// float power-of-two pre-scale of the MFMA path at +16].
constexpr int64_t kLinearTail = 256;
constexpr int64_t kLinearWscOff = 16;

// Largest |q| the MFMA path multiplies a scale by (affine codes recentred to
// u - 2^(b-1)); its power-of-two pre-scale keeps q*s inside f16 range.
__host__ __device__ inline int qtype_qmax(int qt) {
  switch (qt) {
    case QMOE_QTYPE_SYM_INT4: return 8;
    case QMOE_QTYPE_SYM_INT2: return 2;
    case QMOE_QTYPE_TERNARY: return 1;
    case QMOE_QTYPE_AFFINE_INT2: return 2;
    default: return 8;
  }
}

// Affine formats on the MFMA path keep per-row block sums in LDS.
constexpr int kGroupedMaxAffineBlocks = 80;

// ------------------------------------------------------------------ routing
// Device-side routing results, carved from the workspace.
struct RouteBufs {
  int32_t *ids;        // [T*k]
  float *w;            // [T*k]
  int32_t *counts;     // [E]
  int32_t *offsets;    // [E+1]
  int32_t *row_list;   // [T*k]   slot ids grouped by expert
  int32_t *slot_pos;   // [T*k]   inverse of row_list
  int32_t *token_of;   // [T*k]   token of the row at each expert-sorted position
  int32_t *active;     // [E]     experts with count > 0, ascending
  int32_t *num_active; // [1]
  int4 *slot_info;     // [max_slots] {expert, rows, first position, 0}; rows = 0 past num_active
  int4 *tile_info;     // [max_tiles] {expert, first position, rows (<= tile), tiles}; rows = 0 past the end
  int32_t *range_base; // [kPlaceRanges][E] first row_list position of each slot range's rows of each expert
};
// Contiguous slot ranges whose rows the expand kernel counts and a placing
// kernel (one workgroup per range) writes into the row list.
constexpr int kPlaceRanges = 64;
constexpr int kPlaceMinSlots = 4096;  // routed slots from which that ranged sort runs (fewer: one workgroup)

struct RouteArgs {
  const float *logits;
  int T, E, k;
  RouteBufs r;
  int topk_in_expand;  // 1: the expand kernel also performs top-k (small T)
  int max_slots;       // entries of slot_info to fill
  int32_t *zero_buf;   // optional int buffer cleared by the expand kernel
  int zero_len;
  int tile_rows;       // rows per grouped-path tile (0: no tile list)
  int max_tiles;       // entries of tile_info to fill
  int softmax_all;     // 1: weights are the selected entries of the softmax over all E logits
};

// -------------------------------------------------------------------- GEMV
// kEpiSwiGLU: FC1 -> h (bf16 hi + lo parts, optional fp32 copy);
// kEpiDown: FC2 -> per-slot fp32 o; with top-1 routing the combine is a
// single product and y is written directly;
// kEpiStoreAct: dense rows -> y in the activation dtype.
// kEpiSwiGLURouted: kEpiSwiGLU for small decode batches (T * k <=
// kFc1RouteMaxSlots) whose workgroups route the tokens themselves (no
// routing kernel); workgroup 0 also writes the routing lists for FC2, the
// combine and the diagnostics.
// kEpiDownCat: FC2 of one token with k > 1 as one GEMV over the concatenated
// k expert matrices (the routing weight folded into each block's scale), so
// y is written directly and no combine follows.
enum GemvEpilogue { kEpiSwiGLU = 0, kEpiDown = 1, kEpiStoreAct = 2, kEpiSwiGLURouted = 3, kEpiDownCat = 4 };
// Input of the FC1 epilogues (the in_f16 argument of launch_gemv): 0 bf16
// rows, 1 f16 rows, kGemvInSplitF32 f32 rows given as bf16 hi + lo parts.
constexpr int kGemvInSplitF32 = 2;
constexpr int kFc1RouteMaxSlots = 16;  // <= 64 (one slot per lane of the expand)

struct GemvArgs {
  // weights
  const uint8_t *w;        // matrix section base (expert 0)
  int64_t expert_stride;
  int64_t scales_off;
  int64_t N, K, RG, NC, NKT, nblk;
  int qtype, sdtype;
  // rows: routed (slot_info / token_of) or dense (M rows)
  const int4 *slot_info;
  const int32_t *token_of, *row_list;
  int top_k;               // kEpiDown: 1 = write y itself (one expert per token), else o
  int dense_M;             // >0: dense rows 0..M-1, expert 0, no routing
  // input activations as 16-bit pairs; parts = 1 (x) or 2 (hi, lo)
  const uint32_t *in;
  int64_t in_row_pairs;    // row stride in 32-bit pairs
  int64_t in_part_stride;  // in pairs: part 1 of row p at in + p*in_row_pairs + in_part_stride
  int in_gather_token;     // 1: input row = token_of[p] (FC1); 0: input row = p
  // outputs
  float *out_f32;          // kEpiDown: o [p][N]
  uint16_t *out_act;       // kEpiStoreAct: [m][N]; kEpiDown with top-1: y [t][N]
  uint16_t *h_hi, *h_lo;   // kEpiSwiGLU: [p][N/2] bf16 parts of h
  float *h_dbg;            // kEpiSwiGLU: optional [slot][N/2] fp32 ([slot][N] with relu)
  int relu;                // kEpiSwiGLU: the FC1 rows are single ReLU channels, h = max(a, 0)
  int sw_custom;           // kEpiSwiGLU (EXT instances): configurable SwiGLU with the next three
  float sw_alpha, sw_beta, sw_limit;
  const uint16_t *bias;    // kEpiSwiGLU, kEpiDown: optional per-expert output bias [E][N] in act_dtype
  int act_dtype;           // activation dtype of out_act and bias
  const float *route_w;    // kEpiDown: routing weights [T*k]
  // kEpiSwiGLURouted: router logits [T][E] and the routing outputs
  const float *logits;
  int route_T, route_E, route_k, route_max_slots;
  int route_softmax_all;   // kEpiSwiGLURouted (EXT instances): as RouteArgs::softmax_all
  RouteBufs route;
  int cat_stage;           // kEpiDownCat: LDS holds the token's h rows after the reduction buffer
  int h_by_slot;           // kEpiSwiGLU(Routed): h rows at the flat slot index, not the sorted position (the
                           // concatenated FC2 of one token reads them)
};

// Rows per GEMV launch: one 16-row MFMA tile for routed experts, two for
// dense inputs.
constexpr int kGemvMaxRowsDense = 32;
constexpr int kGemvMaxWaves = 8;
constexpr int kGemvCatMaxWaves = 16;  // concatenated FC2: k x (waves per expert) <= 16
constexpr int kCatDeep = 8;           // concatenated FC2: k-tiles per wave requested at once
constexpr int kCatStagePer = 4;       // concatenated FC2: 16-B pieces of h per thread staged in LDS
// Concatenated FC2: the token's h rows (k slots, hi + lo parts of K bf16)
// staged in LDS after the reduction buffer.
inline size_t gemv_cat_stage_bytes(int k, int64_t K) { return (size_t)k * 2 * (size_t)K * 2; }

// Dynamic LDS of one GEMV workgroup: the cross-wave partial sums of the
// tn n-tiles x row tiles x accumulator elements x 64 lanes.
inline int gemv_row_tiles(int rows, int epilogue) { return (epilogue == kEpiStoreAct && rows > 16) ? 2 : 1; }
inline size_t gemv_lds_bytes(int rows, int epilogue, int waves, int tn) {
  const int mt = gemv_row_tiles(rows, epilogue), mr = rows > 1 ? 4 : 1;
  return (size_t)waves * tn * (size_t)mt * (size_t)mr * kLanes * sizeof(float);
}

constexpr size_t kGemvLdsLimit = 64 * 1024;

// Host launchers (defined in the kernel translation units).
hipError_t launch_prepack_matrix(const MatLayout &L, int E, const uint8_t *codes,
                                 const uint16_t *scales, const uint16_t *biases, uint8_t *dst,
                                 uint32_t *err_word, hipStream_t s);
// The scale (and bias) section alone, codes untouched.
hipError_t launch_prepack_scales(const MatLayout &L, int E, const uint16_t *scales, const uint16_t *biases,
                                 uint8_t *dst, hipStream_t s);
hipError_t launch_unpack_matrix(const MatLayout &L, int E, const uint8_t *src, int8_t *codes_out,
                                hipStream_t s);
hipError_t launch_route(const RouteArgs &a, hipStream_t s);
// rows: bound on the rows of any expert (or dense M), <= kGemvMaxRowsDense;
// waves: waves per workgroup (K split); tn: 16-row n-tiles per wave (1 or 4).
hipError_t launch_gemv(const GemvArgs &a, int epilogue, int in_f16, int rows, int waves, int tn, int block,
                       int grid_slots, hipStream_t s);
// Resident workgroups per compute unit of that GEMV kernel (0 if the runtime
// cannot tell).
int gemv_blocks_per_cu(int qtype, int epilogue, int in_f16, int rows, int waves, int tn, int block);
hipError_t launch_combine(const float *o, const int32_t *slot_pos, const float *w, int T, int k,
                          int H, int act_dtype, void *y, hipStream_t s);
// Streaming read of `bytes` (a multiple of 16) over `cus` x 8 workgroups.
hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int cus, hipStream_t s);
// f32 rows -> bf16 hi (RNE of x) and lo (RNE of the remainder) rows.
hipError_t launch_split_f32(const float *x, int64_t n, uint16_t *hi, uint16_t *lo, hipStream_t s);

// ------------------------------------------------------ gathered channels
// Channel-packed buffer (per matrix, experts one after another, 256-B
// aligned sections): FC1 rows [E][2I][H*b/8] in the canonical byte order and
// their scales [E][2I][H/B]; the channel-major down projection [E][I][H*b/8]
// and its scales [E][I][H/B].
// Base-3 rows (both matrices TERNARY_B3): the rows are block records with the
// scales inside them, and the scale sections are empty.
struct ChanLayout {
  bool b3;
  int64_t fc1_row_bytes, dn_row_bytes;
  int64_t fc1_off, fc1_sc_off, dn_off, dn_sc_off, total;
  static ChanLayout make(const qmoe_layer_desc &d) {
    ChanLayout L{};
    const int64_t E = d.num_experts, H = d.hidden, I = d.inter;
    L.b3 = d.fc1.qtype == QMOE_QTYPE_TERNARY_B3;
    L.fc1_row_bytes = L.b3 ? (H / d.fc1.block) * b3_record_bytes(d.fc1.block) : H * qtype_bits(d.fc1.qtype) / 8;
    L.dn_row_bytes = L.b3 ? (H / d.fc2.block) * b3_record_bytes(d.fc2.block) : H * qtype_bits(d.fc2.qtype) / 8;
    const int64_t sc1 = L.b3 ? 0 : E * 2 * I * (H / d.fc1.block) * 2;
    const int64_t sc2 = L.b3 ? 0 : E * I * (H / d.fc2.block) * 2;
    L.fc1_off = kHeaderBytes;
    L.fc1_sc_off = L.fc1_off + align_up(E * 2 * I * L.fc1_row_bytes, kAlign);
    L.dn_off = L.fc1_sc_off + align_up(sc1, kAlign);
    L.dn_sc_off = L.dn_off + align_up(E * I * L.dn_row_bytes, kAlign);
    L.total = L.dn_sc_off + align_up(sc2, kAlign);
    return L;
  }
};

constexpr int kChanGroupEntries = 16;  // list entries per workgroup (partial sums per token: k C / 16)
constexpr int kChanMaxHidden = 4096;
constexpr int kChanMaxHiddenB3 = 2048;  // base-3 rows

struct ChanArgs {
  const uint8_t *fc1, *fc1_scales;
  int64_t fc1_row_bytes;
  int fc1_bits, fc1_block, fc1_sf16, fc1_zp;
  const uint8_t *dn, *dn_scales;
  int64_t dn_row_bytes;
  int dn_bits, dn_block, dn_sf16, dn_zp;
  int b3;                   // both matrices base-3 block records (row bytes: records)
  int T, E, k, C, I, H;
  int groups;               // ceil(k * C / kChanGroupEntries) list groups per token
  const uint16_t *x;        // [T][H], 16-byte aligned
  int x_f16;
  const float *logits;      // [T][E]
  const int32_t *channels;  // [T][k][C]
  float *partial;           // [T][groups][H]
  uint16_t *y;
};
hipError_t launch_channels(const ChanArgs &a, hipStream_t s);
// Canonical base-3 rows [rows][(K/B) ceil(B/5)] and scales [rows][K/B] ->
// block records; counts the invalid bytes into *count.
hipError_t launch_pack_b3_records(const uint8_t *codes, const uint16_t *scales, int64_t rows, int64_t K, int block,
                                  uint8_t *dst, uint32_t *count, hipStream_t s);
// Counts ternary fields holding the invalid value 3 in `bytes` bytes.
hipError_t launch_count_invalid_ternary(const uint8_t *p, int64_t bytes, uint32_t *count, hipStream_t s);

// ----------------------------------------------------------- grouped MFMA
// Shape of a grouped workgroup tile: MI 16-row MFMA row tiles (TM = 16 MI
// rows), NJ 16-column slices per wave, NW waves (16 NJ NW outputs per tile,
// all waves sharing the staged activation tile) and KT k per staged
// activation tile.  Affine formats keep per-row block
// sums of the activations in LDS, laid out for 64-row tiles; the other
// formats take the shapes below (compile-time tuning constants).
#ifndef QMOE_GROUPED_MI
#define QMOE_GROUPED_MI 8
#endif
#ifndef QMOE_GROUPED_NJ16
#define QMOE_GROUPED_NJ16 2
#endif
#ifndef QMOE_GROUPED_KT16
#define QMOE_GROUPED_KT16 64
#endif
#ifndef QMOE_GROUPED_NJ32
#define QMOE_GROUPED_NJ32 2
#endif
#ifndef QMOE_GROUPED_KT32
#define QMOE_GROUPED_KT32 64
#endif
// A fragments read ahead of the MFMAs that use them, plus one: 3 for the
// 128-row tiles of 16-bit rows (FC1: 489 against 506 us on the mixed
// INT2/INT4 prefill), 2 for the others (FC2's two h parts spill with 3)
#ifndef QMOE_GROUPED_AD
#define QMOE_GROUPED_AD 2
#endif
#ifndef QMOE_GROUPED_AD16
#define QMOE_GROUPED_AD16 3
#endif
#ifndef QMOE_GROUPED_NW16
#define QMOE_GROUPED_NW16 8
#endif
#ifndef QMOE_GROUPED_NW32
#define QMOE_GROUPED_NW32 8
#endif
constexpr int kTileM = 64;  // rows per grouped tile with an affine matrix

struct GroupedShape {
  int mi, nj, kt, nw;  // nw: waves per workgroup, which share the staged activation tile
};
// in_f32: the shape of FC2 (fp32 input staged as f16 hi + lo parts, fp32
// per-slot output); FC1 and the dense matrix take the other shape whatever
// their input.  The 64-row shape (affine formats, and a non-affine matrix
// whose layer has an affine one):
__host__ __device__ constexpr GroupedShape grouped_shape_64(bool in_f32) {
  return GroupedShape{4, in_f32 ? 4 : 2, in_f32 ? 64 : 128, 4};
}
// The shape of the other layers:
__host__ __device__ constexpr GroupedShape grouped_shape_main(bool in_f32) {
  return GroupedShape{QMOE_GROUPED_MI, in_f32 ? QMOE_GROUPED_NJ32 : QMOE_GROUPED_NJ16,
                      in_f32 ? QMOE_GROUPED_KT32 : QMOE_GROUPED_KT16, in_f32 ? QMOE_GROUPED_NW32 : QMOE_GROUPED_NW16};
}
// Rows per grouped tile of a call (FC1 and FC2 share the tile list).
inline int grouped_tile_rows(bool any_affine) { return any_affine ? kTileM : 16 * QMOE_GROUPED_MI; }
// The shape one matrix runs with for those tile rows.
inline GroupedShape grouped_shape(bool affine, int tile_rows, bool in_f32) {
  return (!affine && tile_rows == 16 * QMOE_GROUPED_MI) ? grouped_shape_main(in_f32) : grouped_shape_64(in_f32);
}

enum GroupedEpilogue { kGEpiSwiGLU = 0, kGEpiStoreF32 = 1, kGEpiStoreAct = 2 };

struct GroupedArgs {
  const uint8_t *w;        // matrix section base (expert 0)
  int64_t expert_stride, scales_off;
  int64_t N, K, RG, NC, NKT, nblk;
  int qtype, sdtype, block, bpk;
  const float *wsc;        // [E] power-of-two weight pre-scale
  // rows
  const int4 *tile_info;   // routed: {expert, first position, rows, number of tiles}
  int tile_rows;           // rows per tile: kTileM or kTileMWide (routed: as the tile list)
  int dense_M;             // > 0: dense rows, tiles of tile_rows over M
  const int32_t *token_of; // routed FC1: input row of position p
  int in_gather_token;
  // input: 16-bit rows (in_f32 = 0, dtype in_f16), fp32 rows (in_f32 = 1),
  // or f16 rows already multiplied by their power-of-two scale (in_scaled = 1)
  const void *in;
  int in_f32, in_f16, in_scaled;
  int in_split;              // FC2: fp32 rows already split into scaled f16 parts, [hi 8][lo 8] per 8 k (non-affine)
  int64_t in_row_elems;
  const float *in_rowsc;   // 16-bit input: power-of-two scale per input row
  const uint32_t *in_rowmax; // fp32 input: |max| bits per row (scale derived)
  // outputs
  float *out_f32;          // kGEpiSwiGLU: h [p][N/2]; kGEpiStoreF32: o [p][N]
  uint32_t *out_rowmax;    // kGEpiSwiGLU: |max| bits of h per row (atomicMax), zero on entry
  uint16_t *out_act;       // kGEpiStoreAct: y [m][N]
  const uint16_t *bias;    // routed: optional per-expert output bias [E][N] in act_dtype
  int act_dtype;           // activation dtype of out_act and bias
  float *h_dbg;            // optional fp32 copy of h in slot order
  int relu;                // kGEpiSwiGLU: h = max(a, 0) per row instead of SwiGLU pairs
  int sw_custom;           // kGEpiSwiGLU: configurable SwiGLU with the next three
  float sw_alpha, sw_beta, sw_limit;
  const int32_t *row_list;
};

hipError_t launch_grouped(const GroupedArgs &a, int epilogue, int grid_tiles, hipStream_t s);
// Per-row power of two of the f16 A operand; with xs non-null, also the
// scaled rows as f16 (exact: x * 2^r of a bf16/f16 x below 2^14).
hipError_t launch_rowscale(const void *x, int rows, int64_t K, int in_f16, float *rowsc, uint16_t *xs,
                           hipStream_t s);
// Bits of max |x| per fp32 row (K a multiple of 4, rows 16-B aligned).
hipError_t launch_rowmax_f32(const float *x, int rows, int64_t K, uint32_t *rowmax, hipStream_t s);
// fp32 rows [rows][K] (K a multiple of 8) -> in place, per 8 k, [hi 8][lo 8]
// f16 parts of the row times its power of two from rowmax
hipError_t launch_split_rows(float *h, int rows, int64_t K, const uint32_t *rowmax, hipStream_t s);
hipError_t launch_wscale(const MatLayout &L, int E, const uint8_t *mat, float *wsc, hipStream_t s);

// ---------------------------------------------------------------- launches
// Stage timing: while the calling thread has stage events set, every kernel
// goes through hipExtLaunchKernel, which stamps `start` with the begin
// timestamp of the stage's first kernel and `stop` with the end timestamp of
// each kernel (the last kernel's stays), the dispatch timestamps a kernel
// trace reads.  Without events the launch is a plain hipLaunchKernel.
struct StageEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool started = false;
};
StageEvents &stage_events();  // per host thread

inline hipError_t launch_raw(const void *fn, dim3 grid, dim3 block, void **argv, size_t lds, hipStream_t s) {
  StageEvents &ev = stage_events();
  if (ev.stop == nullptr) return hipLaunchKernel(fn, grid, block, argv, lds, s);
  hipEvent_t st = ev.started ? nullptr : ev.start;
  ev.started = true;
  return hipExtLaunchKernel(fn, grid, block, argv, lds, s, st, ev.stop, 0);
}

// Typed launch: the arguments are converted to the kernel's parameter types
// before their addresses are handed to the runtime.
template <typename... P, typename... A>
inline hipError_t qlaunch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A &&...args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> t(static_cast<P>(std::forward<A>(args))...);
  void *argv[sizeof...(P) > 0 ? sizeof...(P) : 1];
  std::apply([&](auto &...x) {
    int i = 0;
    ((argv[i++] = static_cast<void *>(&x)), ...);
  }, t);
  return launch_raw(reinterpret_cast<const void *>(kernel), grid, block, argv, lds, s);
}

}  // namespace qmoe
