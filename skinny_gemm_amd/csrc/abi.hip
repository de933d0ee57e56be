// abi.hip -- the extern "C" boundary: validation, workspace carving, launch
// planning and sequencing.  No allocation, no synchronisation on the forward
// path; every check runs before the first launch.
//
// Problem statement followed (onnxruntime pull request 33005, Description and
// Current Scope): cached prepacked weights, an aligned per-call workspace
// ordered on the stream, FP16/BF16 activations, dimensions divisible by 64,
// at most 256 experts, bounded int-sized routed-row counts, and an explicit
// error instead of a silent fallback for anything outside that scope.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

#include "qmoe_internal.h"

using namespace qmoe;

namespace qmoe {
StageEvents &stage_events() {
  thread_local StageEvents ev;
  return ev;
}
}  // namespace qmoe

namespace {

thread_local std::string g_last_error;

qmoe_status fail(qmoe_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

qmoe_status ok() { return QMOE_OK; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

qmoe_status check_matrix(const qmoe_qmatrix_desc &m, const char *name, int64_t rows, int64_t cols) {
  if (m.reserved != 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "%s: reserved field must be 0", name);
  if (m.qtype < QMOE_QTYPE_SYM_INT4 || m.qtype > QMOE_QTYPE_TERNARY_B3)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: unknown qtype %d", name, m.qtype);
  if (m.scale_dtype != QMOE_DTYPE_BF16 && m.scale_dtype != QMOE_DTYPE_F16)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: scale dtype %d not supported (bf16 or f16)", name,
                m.scale_dtype);
  if (rows >= 0 && (m.rows != rows || m.cols != cols))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "%s: shape [%lld][%lld] but the layer needs [%lld][%lld]",
                name, (long long)m.rows, (long long)m.cols, (long long)rows, (long long)cols);
  if (m.rows <= 0 || m.cols <= 0)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "%s: non-positive shape", name);
  if (m.block != 64 && m.block != 128)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: block %d not supported (64 or 128)", name, m.block);
  if (m.rows % 64 != 0 || m.cols % 64 != 0)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: dimensions must be multiples of 64", name);
  if (m.cols % m.block != 0)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "%s: cols %lld not a multiple of block %d", name,
                (long long)m.cols, m.block);
  if (m.rows > (int64_t)1 << 30 || m.cols > (int64_t)1 << 20)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: dimensions beyond the supported range", name);
  return ok();
}

// channels: the gathered-channel calls, the only ones that take base-3 rows.
qmoe_status check_layer(const qmoe_layer_desc *d, bool channels = false) {
  if (!d) return fail(QMOE_ERR_INVALID_ARGUMENT, "null layer descriptor");
  if (d->num_experts < 1) return fail(QMOE_ERR_INVALID_ARGUMENT, "num_experts must be >= 1");
  if (d->num_experts > kMaxExperts)
    return fail(QMOE_ERR_UNSUPPORTED, "num_experts %d > %d", d->num_experts, kMaxExperts);
  if (d->hidden <= 0 || d->inter <= 0)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "hidden and inter must be positive");
  if (d->act_dtype != QMOE_DTYPE_BF16 && d->act_dtype != QMOE_DTYPE_F16 && d->act_dtype != QMOE_DTYPE_F32)
    return fail(QMOE_ERR_UNSUPPORTED, "activation dtype %d not supported (bf16, f16 or f32)", d->act_dtype);
  if (d->activation != QMOE_ACT_SWIGLU && d->activation != QMOE_ACT_RELU)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "activation %d is not a qmoe_activation value", d->activation);
  if (d->reserved != 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "layer reserved field must be 0");
  const int64_t fc1_rows = d->activation == QMOE_ACT_RELU ? (int64_t)d->inter : 2 * (int64_t)d->inter;
  qmoe_status st = check_matrix(d->fc1, "fc1", fc1_rows, d->hidden);
  if (st == QMOE_OK) st = check_matrix(d->fc2, "fc2", d->hidden, d->inter);
  if (st != QMOE_OK) return st;
  if (!channels && (d->fc1.qtype == QMOE_QTYPE_TERNARY_B3 || d->fc2.qtype == QMOE_QTYPE_TERNARY_B3))
    return fail(QMOE_ERR_UNSUPPORTED, "base-3 ternary rows are read by the gathered-channel calls only");
  return ok();
}

qmoe_status check_tokens(const qmoe_layer_desc *d, int32_t T, int32_t top_k) {
  if (T < 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "T must be >= 0");
  if (top_k < 1 || top_k > d->num_experts)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "top_k %d outside [1, E=%d]", top_k, d->num_experts);
  if (top_k > kMaxTopK) return fail(QMOE_ERR_UNSUPPORTED, "top_k %d > %d", top_k, kMaxTopK);
  if ((int64_t)T * top_k > INT32_MAX)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "T * top_k overflows int32");
  return ok();
}

// ------------------------------------------------------------- workspace
struct Carve {
  int64_t off = 0;
  int64_t take(int64_t bytes) {
    int64_t o = off;
    off += align_up(bytes > 0 ? bytes : 1, kAlign);
    return o;
  }
};

// Upper bound of the grouped tiles of S routed rows over E experts in tiles
// of tm rows (one partial tile per active expert at most).  The workspace
// holds the bound of the smallest tile, so it does not depend on the choice.
inline int64_t grouped_max_tiles(int64_t S, int E, int tm = kTileM) {
  const int64_t t = (S + tm - 1) / tm + std::min<int64_t>(E, S);
  return (t + 7) / 8 * 8;  // a multiple of 8 lets the kernel spread tiles over the XCDs
}

struct RouteWs {
  int64_t ids, w, counts, offsets, row_list, slot_pos, token_of, active, num_active, slot_info, tile_info,
      range_base, end;
  static RouteWs make(Carve &c, int64_t S, int E) {
    RouteWs r;
    r.ids = c.take(S * 4);
    r.w = c.take(S * 4);
    r.counts = c.take((int64_t)E * 4);
    r.offsets = c.take(((int64_t)E + 1) * 4);
    r.row_list = c.take(S * 4);
    r.slot_pos = c.take(S * 4);
    r.token_of = c.take(S * 4);
    r.active = c.take((int64_t)E * 4);
    r.num_active = c.take(4);
    r.slot_info = c.take((int64_t)E * 16);
    r.tile_info = c.take(grouped_max_tiles(S, E) * 16);
    r.range_base = c.take((int64_t)kPlaceRanges * E * 4);
    r.end = c.off;
    return r;
  }
  RouteBufs bind(uint8_t *ws) const {
    RouteBufs b;
    b.ids = (int32_t *)(ws + ids);
    b.w = (float *)(ws + w);
    b.counts = (int32_t *)(ws + counts);
    b.offsets = (int32_t *)(ws + offsets);
    b.row_list = (int32_t *)(ws + row_list);
    b.slot_pos = (int32_t *)(ws + slot_pos);
    b.token_of = (int32_t *)(ws + token_of);
    b.active = (int32_t *)(ws + active);
    b.num_active = (int32_t *)(ws + num_active);
    b.slot_info = (int4 *)(ws + slot_info);
    b.tile_info = (int4 *)(ws + tile_info);
    b.range_base = (int32_t *)(ws + range_base);
    return b;
  }
};

// GEMV path: h as bf16 hi/lo parts; grouped path: h fp32 + per-row |max|
// and the per-token activation scales.  Both paths write o [S][H] fp32.
struct MoeWs {
  RouteWs route;
  int64_t h_hi, h_lo, h32, hmax, xsc, xs16, x_hi, x_lo, o, total;
  static MoeWs make(const qmoe_layer_desc &d, int32_t T, int32_t k, bool grouped) {
    MoeWs w;
    w.x_hi = w.x_lo = 0;
    Carve c;
    const int64_t S = (int64_t)T * k;
    w.route = RouteWs::make(c, S, d.num_experts);
    if (grouped) {
      w.h_hi = w.h_lo = 0;
      w.h32 = c.take(S * d.inter * 4);
      w.hmax = c.take(S * 4);
      w.xsc = c.take((int64_t)T * 4);
      w.xs16 = c.take((int64_t)T * d.hidden * 2);
    } else {
      w.h_hi = c.take(S * d.inter * 2);
      w.h_lo = c.take(S * d.inter * 2);
      w.h32 = w.hmax = w.xsc = w.xs16 = 0;
      // f32 activations: x as bf16 hi + lo rows (the FC1 A operand)
      w.x_hi = d.act_dtype == QMOE_DTYPE_F32 ? c.take((int64_t)T * d.hidden * 2) : 0;
      w.x_lo = d.act_dtype == QMOE_DTYPE_F32 ? c.take((int64_t)T * d.hidden * 2) : 0;
    }
    w.o = c.take(S * d.hidden * 4);
    w.total = c.off;
    return w;
  }
  static int64_t worst(const qmoe_layer_desc &d, int32_t T, int32_t k) {
    return std::max(make(d, T, k, false).total, make(d, T, k, true).total);
  }
};

// ------------------------------------------------------------------ plan
constexpr size_t kLdsLimit = kGemvLdsLimit;

// Waves on the chip that a GEMV launch aims for when the kernel's occupancy
// is unknown.
constexpr int64_t kGemvTargetWaves = 4096;

// Compute units of the current device (256 on MI355X when there is none).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

// Shape of a GEMV launch.  Waves per workgroup of the split-K GEMV (at most one per k-tile and
// kGemvMaxWaves).  With the kernel's occupancy known, the choice minimises
// the critical path: rounds of resident workgroups x k-tiles per wave (ties
// to fewer waves).  Wave counts that do not divide evenly over the 4 SIMDs
// of a compute unit (3, 5, 6, 7) leave one SIMD with more waves of every
// workgroup; such a count is a candidate only when it gives every wave a
// single k-tile (the shortest critical path).  Without the occupancy (no device),
// enough waves on the chip to cover HBM latency.  nwg: workgroups of the
// launch; rows: its row bound.
struct GemvShape {
  int waves, tn;
};

GemvShape pick_gemv(int64_t nwg, const MatLayout &L, int rows, int epilogue, int in_f16) {
  const int64_t kmax = std::min<int64_t>(kGemvMaxWaves, L.NKT);
  const int64_t cus = device_cus();
  // four n-tiles per wave unless that leaves compute units idle
  const int tn = nwg < cus ? 1 : 4;
  nwg *= 4 / tn;
  int best = 0;
  int64_t best_cost = 0;
  for (int ks = 1; ks <= kmax; ++ks) {
    if (gemv_lds_bytes(rows, epilogue, ks, tn) > kLdsLimit) break;
    const bool balanced = (ks & (ks - 1)) == 0;
    if (!balanced && ks != L.NKT) continue;
    const int per_cu = gemv_blocks_per_cu(L.qtype, epilogue, in_f16, rows, ks, tn, L.block);
    if (per_cu <= 0) {
      best = 0;
      break;
    }
    const int64_t rounds = (nwg + cus * per_cu - 1) / (cus * per_cu);
    const int64_t cost = rounds * ((L.NKT + ks - 1) / ks);
    if (best == 0 || cost < best_cost) {
      best = ks;
      best_cost = cost;
    }
  }
  if (best > 0) {
    // FC1 launches that fill the chip (four n-tiles a wave) keep at least 4
    // k-tiles a wave: the per-wave fixed work (routing prologue, 64-row
    // SwiGLU epilogue, the LDS reduction) outweighs the shorter chain there
    // (DeepSeek-V2-Lite-shaped decode, 16 k-tiles: FC1 at 4 waves measured
    // 4-13% faster than at 8)
    if (tn == 4 && (epilogue == kEpiSwiGLU || epilogue == kEpiSwiGLURouted))
      while (best > 1 && L.NKT / best < 4) best /= 2;
    return {best, tn};
  }
  int64_t ks = (kGemvTargetWaves + nwg - 1) / std::max<int64_t>(nwg, 1);
  ks = std::max<int64_t>(1, std::min<int64_t>(ks, kmax));
  while (ks > 1 && gemv_lds_bytes(rows, epilogue, (int)ks, tn) > kLdsLimit) --ks;
  return {(int)ks, tn};
}

struct Plan {
  int path;
  int mmax, mmax1, mmax2, ks1, ks2, tn1, tn2, max_active, max_tiles, tile_rows;
  int route_fused;
  int fc1_routes;  // GEMV path: FC1 routes the tokens itself (no routing kernel)
  int fc2_cat;     // GEMV path, one token, k > 1: FC2 over the k experts' concatenated K writes y (no combine)
  int cat_stage;   // fc2_cat: the token's h rows fit LDS beside the reduction (the one-request weight path)
  bool softmax_all;  // unnormalised top-k weights, computed by the routing top-k
  int launches;
  std::string kernels;
};

// FC1 input mode of the GEMV for an activation dtype.
int gemv_in_mode(int act_dtype) {
  return act_dtype == QMOE_DTYPE_F32 ? kGemvInSplitF32 : act_dtype == QMOE_DTYPE_F16 ? 1 : 0;
}

// Whether the grouped kernels take this layer: affine formats need at most
// kGroupedMaxAffineBlocks blocks per row (their per-row block sums live in
// LDS).
bool grouped_supported(const qmoe_layer_desc &d) {
  const MoeLayout L = MoeLayout::make(d);
  return !((L.fc1.affine && L.fc1.nblk > kGroupedMaxAffineBlocks) ||
           (L.fc2.affine && L.fc2.nblk > kGroupedMaxAffineBlocks));
}

// Largest tile a call may run as one pass: the GEMV path's row bound when
// the call is pinned to it or the layer has no grouped path.
int32_t path_row_bound(const qmoe_layer_desc &d, int path_req) {
  if (path_req == QMOE_PATH_GEMV || (path_req == QMOE_PATH_AUTO && !grouped_supported(d))) return kGemvMaxRows;
  return INT32_MAX;
}

qmoe_status make_plan(const qmoe_layer_desc &d, int32_t T, int32_t k, int path_req, bool softmax_all, bool fc2_bias,
                      Plan &p) {
  const MoeLayout L = MoeLayout::make(d);
  p = Plan{};
  int path = path_req;
  if (path != QMOE_PATH_AUTO && path != QMOE_PATH_GEMV && path != QMOE_PATH_GROUPED)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "unknown path %d", path_req);
  if (path == QMOE_PATH_AUTO)
    path = (T <= kGemvMaxRows || !grouped_supported(d)) ? QMOE_PATH_GEMV : QMOE_PATH_GROUPED;
  if (path == QMOE_PATH_GEMV && T > kGemvMaxRows)
    return fail(QMOE_ERR_UNSUPPORTED, "GEMV path needs T <= %d (got %d)%s", kGemvMaxRows, T,
                path_req == QMOE_PATH_AUTO ? ": this layer has no grouped path, run it in row tiles" : "");
  p.path = path;
  p.max_active = (int)std::min<int64_t>(d.num_experts, (int64_t)T * k);
  const bool f32 = d.act_dtype == QMOE_DTYPE_F32;
  if (path == QMOE_PATH_GROUPED) {
    if (!grouped_supported(d))
      return fail(QMOE_ERR_UNSUPPORTED, "affine formats on the grouped path need K/block <= %d",
                  kGroupedMaxAffineBlocks);
    p.route_fused = (T <= 16) ? 1 : 0;
    p.tile_rows = grouped_tile_rows(L.fc1.affine || L.fc2.affine);
    p.max_tiles = (int)grouped_max_tiles((int64_t)T * k, d.num_experts, p.tile_rows);
    p.softmax_all = softmax_all;
    p.kernels = std::string("route,") + "rowscale,grouped_fc1_" +
                (d.activation == QMOE_ACT_RELU ? "relu" : "swiglu") + (L.fc2.affine ? "" : ",split_h") +
                ",grouped_fc2,combine";
    // routing: the one-workgroup expand (with the top-k up to 16 tokens, else
    // after it), or from kPlaceMinSlots slots top-k, count, expand, place
    p.launches = (p.route_fused ? 1 : (int64_t)T * k >= kPlaceMinSlots ? 4 : 2) + 4 + (L.fc2.affine ? 0 : 1);
    return ok();
  }
  p.route_fused = (T <= 16) ? 1 : 0;
  // a few routed slots: every FC1 workgroup routes them itself (the routing
  // is repeated by every workgroup, so only while it is a small fraction of
  // the work: more slots take the routing kernel)
  p.fc1_routes = ((int64_t)T * k <= kFc1RouteMaxSlots) ? 1 : 0;
  p.max_active = (int)std::min<int64_t>(d.num_experts, (int64_t)T * k);
  p.mmax = p.mmax1 = p.mmax2 = T;  // no expert gets more rows than there are tokens
  const GemvShape g1 = pick_gemv((int64_t)p.max_active * L.fc1.RG, L.fc1, T,
                                 p.fc1_routes ? kEpiSwiGLURouted : kEpiSwiGLU, gemv_in_mode(d.act_dtype));
  // one token with k > 1 (16-bit y, no FC2 bias): FC2 runs over the k
  // matrices end to end, routing weights in the block scales, and writes y
  p.fc2_cat = (T == 1 && k > 1 && d.act_dtype != QMOE_DTYPE_F32 && !fc2_bias) ? 1 : 0;
  MatLayout L2 = L.fc2;
  if (p.fc2_cat) L2.NKT *= k;  // the K split of the concatenated matrices
  const GemvShape g2 = p.fc2_cat ? pick_gemv(L.fc2.RG, L2, T, kEpiDownCat, 0)
                                 : pick_gemv((int64_t)p.max_active * L.fc2.RG, L.fc2, T, kEpiDown, 0);
  p.ks1 = g1.waves;
  p.tn1 = g1.tn;
  p.ks2 = g2.waves;
  // the concatenated FC2 keeps one n-tile a wave: with four its weights and
  // partial sums do not fit the registers (it spills 36-488 B a lane)
  p.tn2 = p.fc2_cat ? 1 : g2.tn;
  // concatenated FC2: the same number of waves on each expert matrix (the
  // most that fit a workgroup of kGemvCatMaxWaves), so that no wave's range
  // crosses from one expert to the next
  if (p.fc2_cat && k <= kGemvCatMaxWaves) {
    const int m = kGemvCatMaxWaves / k;
    if (gemv_lds_bytes(T, kEpiDownCat, k * m, p.tn2) <= kLdsLimit) p.ks2 = k * m;
  }
  p.cat_stage = (p.fc2_cat && p.ks2 % k == 0 &&
                 gemv_lds_bytes(T, kEpiDownCat, p.ks2, p.tn2) + gemv_cat_stage_bytes(k, d.inter) <= kLdsLimit)
                    ? 1
                    : 0;
  // top-1: the down GEMV writes y; otherwise a combine kernel follows
  // the weights of SOFTMAX_ALL replace the routing's weights once the ids
  // exist, before the first reader of the weights (FC2 or the combine)
  p.softmax_all = softmax_all;
  // f32 activations: a split pass first, and y always from the combine
  const bool combine = (k > 1 || f32) && !p.fc2_cat;
  const std::string act = d.activation == QMOE_ACT_RELU ? "relu" : "swiglu";
  p.kernels = std::string(f32 ? "split_x," : "") + (p.fc1_routes ? "route_fc1_" + act : "route,gemv_fc1_" + act) +
              (p.fc2_cat ? ",gemv_fc2_combine" : ",gemv_fc2") + (combine ? ",combine" : "");
  p.launches = (p.fc1_routes ? 2 : 3) + (combine ? 1 : 0) + (f32 ? 1 : 0);
  return ok();
}

qmoe_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(QMOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

GroupedArgs grouped_base(const MatLayout &L, const uint8_t *w, const float *wsc) {
  GroupedArgs g;
  memset(&g, 0, sizeof g);
  g.w = w;
  g.expert_stride = L.stride;
  g.scales_off = L.scales_off;
  g.N = L.N;
  g.K = L.K;
  g.RG = L.RG;
  g.NC = L.NC;
  g.NKT = L.NKT;
  g.nblk = L.nblk;
  g.qtype = L.qtype;
  g.sdtype = L.sdtype;
  g.block = L.block;
  g.bpk = L.bpk;
  g.wsc = wsc;
  return g;
}

qmoe_status copy_diagnostics(const qmoe_layer_desc *desc, const qmoe_forward_opts *opts, const RouteBufs &r,
                             int64_t S, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (opts && opts->ids_out) e = hipMemcpyAsync(opts->ids_out, r.ids, S * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && opts && opts->w_out)
    e = hipMemcpyAsync(opts->w_out, r.w, S * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && opts && opts->counts_out)
    e = hipMemcpyAsync(opts->counts_out, r.counts, (size_t)desc->num_experts * 4, hipMemcpyDeviceToDevice, s);
  return hip_status(e, "diagnostic copies");
}

// The configurable SwiGLU parameters of the call, if any.
template <typename Args>
void set_swiglu(Args &g, const qmoe_forward_opts *opts) {
  g.sw_custom = (opts && opts->swiglu_params == 1) ? 1 : 0;
  g.sw_alpha = g.sw_custom ? opts->swiglu_alpha : 1.f;
  g.sw_beta = g.sw_custom ? opts->swiglu_beta : 0.f;
  g.sw_limit = g.sw_custom ? opts->swiglu_limit : 0.f;
}

GemvArgs gemv_base(const MatLayout &L, const uint8_t *w) {
  GemvArgs g;
  memset(&g, 0, sizeof g);
  g.w = w;
  g.expert_stride = L.stride;
  g.scales_off = L.scales_off;
  g.N = L.N;
  g.K = L.K;
  g.RG = L.RG;
  g.NC = L.NC;
  g.NKT = L.NKT;
  g.nblk = L.nblk;
  g.qtype = L.qtype;
  g.sdtype = L.sdtype;
  return g;
}

}  // namespace

extern "C" {

int32_t qmoe_abi_version(void) { return QMOE_ABI_VERSION; }

const char *qmoe_last_error(void) { return g_last_error.c_str(); }

qmoe_status qmoe_prepacked_size(const qmoe_layer_desc *desc, size_t *bytes) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  *bytes = (size_t)MoeLayout::make(*desc).total;
  return ok();
}

qmoe_status qmoe_prepack(const qmoe_layer_desc *desc, const void *fc1_codes, const void *fc1_scales,
                         const void *fc1_biases, const void *fc2_codes, const void *fc2_scales,
                         const void *fc2_biases, void *dst, size_t dst_bytes, void *stream) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  const MoeLayout L = MoeLayout::make(*desc);
  if (!fc1_codes || !fc1_scales || !fc2_codes || !fc2_scales || !dst)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "null source or destination pointer");
  if (L.fc1.affine != (fc1_biases != nullptr) || L.fc2.affine != (fc2_biases != nullptr))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "biases are required for affine formats and only for them");
  if (!aligned(dst, kAlign)) return fail(QMOE_ERR_INVALID_ARGUMENT, "dst must be 256-byte aligned");
  if (!aligned(fc1_scales, 2) || !aligned(fc2_scales, 2) || (fc1_biases && !aligned(fc1_biases, 2)) ||
      (fc2_biases && !aligned(fc2_biases, 2)))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "scale/bias arrays must be 2-byte aligned");
  if (dst_bytes < (size_t)L.total)
    return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "dst holds %zu bytes, %lld needed", dst_bytes,
                (long long)L.total);
  hipStream_t s = (hipStream_t)stream;
  uint8_t *d = (uint8_t *)dst;
  uint8_t header[kHeaderBytes];
  memset(header, 0, sizeof header);
  const uint64_t magic = kPackMagic;
  memcpy(header, &magic, 8);
  memcpy(header + 8, desc, sizeof(qmoe_layer_desc) < 112 ? sizeof(qmoe_layer_desc) : 112);
  hipError_t e = hipMemcpyAsync(d, header, kHeaderBytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_status(e, "header copy");
  uint32_t *err = (uint32_t *)(d + kErrWordOff);
  e = launch_prepack_matrix(L.fc1, desc->num_experts, (const uint8_t *)fc1_codes,
                            (const uint16_t *)fc1_scales, (const uint16_t *)fc1_biases, d + L.fc1_off, err, s);
  if (e != hipSuccess) return hip_status(e, "prepack fc1");
  e = launch_prepack_matrix(L.fc2, desc->num_experts, (const uint8_t *)fc2_codes,
                            (const uint16_t *)fc2_scales, (const uint16_t *)fc2_biases, d + L.fc2_off, err, s);
  if (e != hipSuccess) return hip_status(e, "prepack fc2");
  e = launch_wscale(L.fc1, desc->num_experts, d + L.fc1_off, (float *)(d + L.wsc_off), s);
  if (e == hipSuccess)
    e = launch_wscale(L.fc2, desc->num_experts, d + L.fc2_off, (float *)(d + L.wsc_off) + desc->num_experts, s);
  if (e != hipSuccess) return hip_status(e, "prepack weight scales");
  uint32_t nbad = 0;
  e = hipMemcpyAsync(&nbad, err, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "prepack error word");
  if (nbad) return fail(QMOE_ERR_INVALID_ARGUMENT, "%u ternary fields hold the invalid value 3", nbad);
  return ok();
}

qmoe_status qmoe_prepack_scales(const qmoe_layer_desc *desc, const void *fc1_scales, const void *fc1_biases,
                                const void *fc2_scales, const void *fc2_biases, void *packed, size_t packed_bytes,
                                void *stream) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  const MoeLayout L = MoeLayout::make(*desc);
  if (!fc1_scales || !fc2_scales || !packed) return fail(QMOE_ERR_INVALID_ARGUMENT, "null scale or packed pointer");
  if (L.fc1.affine != (fc1_biases != nullptr) || L.fc2.affine != (fc2_biases != nullptr))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "biases are required for affine formats and only for them");
  if (!aligned(packed, kAlign)) return fail(QMOE_ERR_INVALID_ARGUMENT, "packed must be 256-byte aligned");
  if (!aligned(fc1_scales, 2) || !aligned(fc2_scales, 2) || (fc1_biases && !aligned(fc1_biases, 2)) ||
      (fc2_biases && !aligned(fc2_biases, 2)))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "scale/bias arrays must be 2-byte aligned");
  if (packed_bytes < (size_t)L.total)
    return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "packed holds %zu bytes, %lld needed", packed_bytes,
                (long long)L.total);
  hipStream_t s = (hipStream_t)stream;
  uint8_t *d = (uint8_t *)packed;
  hipError_t e = launch_prepack_scales(L.fc1, desc->num_experts, (const uint16_t *)fc1_scales,
                                       (const uint16_t *)fc1_biases, d + L.fc1_off, s);
  if (e == hipSuccess)
    e = launch_prepack_scales(L.fc2, desc->num_experts, (const uint16_t *)fc2_scales, (const uint16_t *)fc2_biases,
                              d + L.fc2_off, s);
  if (e == hipSuccess) e = launch_wscale(L.fc1, desc->num_experts, d + L.fc1_off, (float *)(d + L.wsc_off), s);
  if (e == hipSuccess)
    e = launch_wscale(L.fc2, desc->num_experts, d + L.fc2_off, (float *)(d + L.wsc_off) + desc->num_experts, s);
  return e == hipSuccess ? ok() : hip_status(e, "prepack scales");
}

qmoe_status qmoe_workspace_size(const qmoe_layer_desc *desc, int32_t T, int32_t top_k, size_t *bytes) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  st = check_tokens(desc, T, top_k);
  if (st != QMOE_OK) return st;
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  *bytes = (size_t)MoeWs::worst(*desc, T, top_k);
  return ok();
}

// Row tiling under a workspace limit: R = T halved (rounding up) until the
// workspaces of a full tile and of the final partial tile, each on its own
// path, fit within the limit.
struct Tiling {
  int32_t rows = 0, tiles = 0;
  int64_t ws = 0;       // the largest tile workspace
  int launches = 0;     // kernels over all tiles
};

qmoe_status tile_need(const qmoe_layer_desc &d, int32_t T, int32_t k, int path_req, bool softmax_all,
                      bool fc2_bias, int32_t R, Tiling &t) {
  t = Tiling{};
  t.rows = R;
  t.tiles = (int32_t)(((int64_t)T + R - 1) / R);
  const int32_t last = T - (t.tiles - 1) * R;  // in [1, R]
  Plan pf, pl;
  qmoe_status st = make_plan(d, R, k, path_req, softmax_all, fc2_bias, pf);
  if (st == QMOE_OK) st = make_plan(d, last, k, path_req, softmax_all, fc2_bias, pl);
  if (st != QMOE_OK) return st;
  t.ws = std::max(MoeWs::make(d, R, k, pf.path == QMOE_PATH_GROUPED).total,
                  MoeWs::make(d, last, k, pl.path == QMOE_PATH_GROUPED).total);
  t.launches = (t.tiles - 1) * pf.launches + pl.launches;
  return QMOE_OK;
}

// Row tiles of one call: R starts at T and is halved (rounding up) while it
// exceeds the row bound of the path (the GEMV path's 16 rows when the layer
// has no grouped path, or when a call with a workspace limit is pinned to the
// GEMV path), then while a full tile's or the final tile's workspace exceeds
// `limit` (0: no limit).
qmoe_status pick_tiling(const qmoe_layer_desc &d, int32_t T, int32_t k, int path_req, bool softmax_all,
                        bool fc2_bias, int64_t limit, Tiling &t) {
  int32_t R = T;
  const int32_t bound = path_row_bound(d, path_req);
  if (path_req == QMOE_PATH_AUTO || limit > 0)
    while (R > bound) R = (R + 1) / 2;
  for (;;) {
    qmoe_status st = tile_need(d, T, k, path_req, softmax_all, fc2_bias, R, t);
    if (st != QMOE_OK) return st;
    if (limit <= 0 || t.ws <= limit) return QMOE_OK;
    if (R == 1)
      return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "one row needs %lld workspace bytes, the limit is %lld",
                  (long long)t.ws, (long long)limit);
    R = (R + 1) / 2;
  }
}

// A call runs in row tiles when it has a workspace limit, or when the layer
// has no grouped path and the tokens exceed the GEMV path's row bound.
bool call_tiled(const qmoe_layer_desc &d, int32_t T, const qmoe_forward_opts *opts) {
  if (T <= 0) return false;
  if (opts && opts->workspace_limit > 0) return true;
  const int path_req = opts ? opts->path : QMOE_PATH_AUTO;
  return path_req == QMOE_PATH_AUTO && T > path_row_bound(d, path_req);
}

qmoe_status qmoe_forward_plan(const qmoe_layer_desc *desc, int32_t T, int32_t top_k,
                              const qmoe_forward_opts *opts, qmoe_plan *plan) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  st = check_tokens(desc, T, top_k);
  if (st != QMOE_OK) return st;
  if (!plan) return fail(QMOE_ERR_INVALID_ARGUMENT, "null plan output");
  const bool softmax_all = opts && opts->topk_weights == QMOE_TOPK_SOFTMAX_ALL;
  if (opts && opts->workspace_limit < 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "negative workspace_limit");
  // with a workspace limit, the plan of a full tile (and the totals over all tiles)
  const bool tiled = call_tiled(*desc, T, opts);
  Tiling tl;
  tl.rows = T;
  tl.tiles = T == 0 ? 0 : 1;
  if (tiled) {
    st = pick_tiling(*desc, T, top_k, opts ? opts->path : QMOE_PATH_AUTO, softmax_all, opts && opts->fc2_bias,
                     opts ? opts->workspace_limit : 0, tl);
    if (st != QMOE_OK) return st;
  }
  Plan p;
  st = make_plan(*desc, tl.rows, top_k, opts ? opts->path : QMOE_PATH_AUTO, softmax_all,
                 opts && opts->fc2_bias, p);
  if (st != QMOE_OK) return st;
  memset(plan, 0, sizeof *plan);
  plan->path = p.path;
  plan->num_launches = T == 0 ? 0 : tiled ? tl.launches : p.launches;
  plan->gemv_mmax = p.mmax;
  plan->gemv_fc1_waves = p.ks1;
  plan->gemv_fc2_waves = p.ks2;
  plan->max_active = p.max_active;
  plan->workspace_bytes = tiled ? tl.ws : MoeWs::make(*desc, T, top_k, p.path == QMOE_PATH_GROUPED).total;
  snprintf(plan->kernels, sizeof plan->kernels, "%s", T == 0 ? "" : p.kernels.c_str());
  plan->row_tile = tl.rows;
  plan->num_tiles = tl.tiles;
  return ok();
}

qmoe_status qmoe_forward_ex(const qmoe_layer_desc *desc, const void *packed, const void *x,
                            const float *logits, int32_t T, int32_t top_k, void *y, void *ws,
                            size_t ws_bytes, void *stream, const qmoe_forward_opts *opts) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  st = check_tokens(desc, T, top_k);
  if (st != QMOE_OK) return st;
  if (opts && (opts->reserved != 0 || opts->reserved2 != 0))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "opts.reserved fields must be 0");
  if (opts && opts->num_events > 0 && !opts->events)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "opts.events is null but num_events > 0");
  if (opts && opts->reserved3 != 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "opts.reserved3 must be 0");
  if (opts && opts->topk_weights != QMOE_TOPK_RENORMALIZED && opts->topk_weights != QMOE_TOPK_SOFTMAX_ALL)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "opts.topk_weights %d is not a qmoe_topk_weights value",
                opts->topk_weights);
  if (opts && opts->workspace_limit < 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "negative workspace_limit");
  if (opts && (opts->fc1_bias || opts->fc2_bias) && desc->act_dtype == QMOE_DTYPE_F32)
    return fail(QMOE_ERR_UNSUPPORTED, "expert biases need 16-bit activations");
  if (opts && opts->swiglu_params != 0) {
    if (opts->swiglu_params != 1)
      return fail(QMOE_ERR_INVALID_ARGUMENT, "opts.swiglu_params must be 0 or 1");
    if (desc->activation != QMOE_ACT_SWIGLU)
      return fail(QMOE_ERR_INVALID_ARGUMENT, "SwiGLU parameters need a SWIGLU layer");
    if (!std::isfinite(opts->swiglu_alpha) || !std::isfinite(opts->swiglu_beta) ||
        !std::isfinite(opts->swiglu_limit) || opts->swiglu_limit < 0.f)
      return fail(QMOE_ERR_INVALID_ARGUMENT, "SwiGLU alpha and beta must be finite, limit finite and >= 0");
  }
  if (T == 0) return ok();
  const bool softmax_all = opts && opts->topk_weights == QMOE_TOPK_SOFTMAX_ALL;
  if (call_tiled(*desc, T, opts)) {
    Tiling tl;
    st = pick_tiling(*desc, T, top_k, opts ? opts->path : QMOE_PATH_AUTO, softmax_all, opts && opts->fc2_bias,
                     opts ? opts->workspace_limit : 0, tl);
    if (st != QMOE_OK) return st;
    if (tl.tiles > 1) {
      // everything a tile could reject is checked here, before the first launch
      if (opts && (opts->counts_out || opts->num_events > 0))
        return fail(QMOE_ERR_UNSUPPORTED, "counts_out and events need a single tile (%d tiles)", tl.tiles);
      if (!packed || !x || !logits || !y || !ws) return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
      if (!aligned(packed, kAlign) || !aligned(ws, kAlign))
        return fail(QMOE_ERR_INVALID_ARGUMENT, "packed and ws must be 256-byte aligned");
      if (!aligned(x, 16) || !aligned(y, 16) || !aligned(logits, 4))
        return fail(QMOE_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned, logits 4-byte aligned");
      if (ws_bytes < (size_t)tl.ws)
        return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %lld needed per tile", ws_bytes,
                    (long long)tl.ws);
      // tiles in order on the stream, sharing the workspace; a tile's rows
      // start at row t0 of x, logits, y and the per-slot diagnostics
      qmoe_forward_opts o{};
      if (opts) o = *opts;
      o.workspace_limit = 0;
      const int64_t H = desc->hidden, E = desc->num_experts, I = desc->inter;
      const int64_t act_bytes = desc->act_dtype == QMOE_DTYPE_F32 ? 4 : 2;
      for (int32_t t0 = 0; t0 < T; t0 += tl.rows) {
        const int32_t n = std::min(tl.rows, T - t0);
        const int64_t s0 = (int64_t)t0 * top_k;
        o.h_out = opts && opts->h_out ? opts->h_out + s0 * I : nullptr;
        o.ids_out = opts && opts->ids_out ? opts->ids_out + s0 : nullptr;
        o.w_out = opts && opts->w_out ? opts->w_out + s0 : nullptr;
        const int64_t xoff = (int64_t)t0 * H * act_bytes;  // bytes: rows of x and y
        st = qmoe_forward_ex(desc, packed, (const uint8_t *)x + xoff, logits + (int64_t)t0 * E, n, top_k,
                             (uint8_t *)y + xoff, ws, ws_bytes, stream, &o);
        if (st != QMOE_OK) return st;
      }
      return ok();
    }
  }
  Plan p;
  st = make_plan(*desc, T, top_k, opts ? opts->path : QMOE_PATH_AUTO, softmax_all, opts && opts->fc2_bias, p);
  if (st != QMOE_OK) return st;
  if (!packed || !x || !logits || !y || !ws)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  if (!aligned(packed, kAlign) || !aligned(ws, kAlign))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "packed and ws must be 256-byte aligned");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(logits, 4))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned, logits 4-byte aligned");
  const MoeWs W = MoeWs::make(*desc, T, top_k, p.path == QMOE_PATH_GROUPED);
  if (ws_bytes < (size_t)W.total)
    return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %lld needed", ws_bytes,
                (long long)W.total);

  hipStream_t s = (hipStream_t)stream;
  uint8_t *wsb = (uint8_t *)ws;
  const MoeLayout L = MoeLayout::make(*desc);
  const uint8_t *pk = (const uint8_t *)packed;
  RouteArgs ra;
  ra.logits = logits;
  ra.T = T;
  ra.E = desc->num_experts;
  ra.k = top_k;
  ra.r = W.route.bind(wsb);
  ra.topk_in_expand = p.route_fused;
  ra.max_slots = p.max_active;
  ra.zero_buf = p.path == QMOE_PATH_GROUPED ? (int32_t *)(wsb + W.hmax) : nullptr;
  ra.zero_len = p.path == QMOE_PATH_GROUPED ? (int)((int64_t)T * top_k) : 0;
  ra.tile_rows = p.path == QMOE_PATH_GROUPED ? p.tile_rows : 0;
  ra.max_tiles = p.max_tiles;
  ra.softmax_all = p.softmax_all ? 1 : 0;
  // optional per-stage events (diagnostic timing): stage i of the plan's
  // stage list stamps events 2i / 2i+1 with the begin of its first kernel
  // and the end of its last (see StageEvents)
  auto ev = [&](int slot) -> hipEvent_t {
    if (!opts || !opts->events || slot >= opts->num_events) return nullptr;
    return (hipEvent_t)opts->events[slot];
  };
  int stage = 0;
  struct StageReset {  // no events stay set past this call, error returns included
    ~StageReset() { stage_events() = StageEvents{}; }
  } stage_reset;
  auto begin = [&]() -> hipError_t {
    hipEvent_t a = ev(2 * stage), b = ev(2 * stage + 1);
    stage_events() = (a && b) ? StageEvents{a, b, false} : StageEvents{};
    return hipSuccess;
  };
  auto end = [&]() -> hipError_t {
    stage_events() = StageEvents{};
    ++stage;
    return hipSuccess;
  };
  hipError_t e = hipSuccess;
  const bool f32 = desc->act_dtype == QMOE_DTYPE_F32;
  uint16_t *x_hi = (uint16_t *)(wsb + W.x_hi), *x_lo = (uint16_t *)(wsb + W.x_lo);
  if (f32 && p.path == QMOE_PATH_GEMV) {  // x as bf16 hi + lo rows for the FC1 GEMV
    e = begin();
    if (e == hipSuccess) e = launch_split_f32((const float *)x, (int64_t)T * desc->hidden, x_hi, x_lo, s);
    if (e == hipSuccess) e = end();
    if (e != hipSuccess) return hip_status(e, "split x");
  }
  const bool fc1_routes = p.path == QMOE_PATH_GEMV && p.fc1_routes;
  if (!fc1_routes) {
    e = begin();
    if (e == hipSuccess) e = launch_route(ra, s);
    if (e == hipSuccess) e = end();
    if (e != hipSuccess) return hip_status(e, "route");
  }

  float *o = (float *)(wsb + W.o);
  if (p.path == QMOE_PATH_GROUPED) {
    float *xsc = (float *)(wsb + W.xsc), *h32 = (float *)(wsb + W.h32);
    uint32_t *hmax = (uint32_t *)(wsb + W.hmax);
    uint16_t *xs16 = (uint16_t *)(wsb + W.xs16);
    const float *wsc = (const float *)(pk + L.wsc_off);
    // fp32 x: the kernel stages each row as f16 hi + lo parts under a power
    // of two from the row's max |x|; 16-bit x: the rows scaled once to f16
    e = begin();
    if (e == hipSuccess)
      e = f32 ? launch_rowmax_f32((const float *)x, T, desc->hidden, (uint32_t *)xsc, s)
              : launch_rowscale(x, T, desc->hidden, desc->act_dtype == QMOE_DTYPE_F16, xsc, xs16, s);
    if (e == hipSuccess) e = end();
    if (e != hipSuccess) return hip_status(e, "rowscale");
    GroupedArgs q1 = grouped_base(L.fc1, pk + L.fc1_off, wsc);
    q1.tile_rows = p.tile_rows;
    q1.tile_info = ra.r.tile_info;
    q1.token_of = ra.r.token_of;
    q1.in_gather_token = 1;
    q1.in_row_elems = desc->hidden;
    if (f32) {
      q1.in = x;
      q1.in_f32 = 1;
      q1.in_rowmax = (const uint32_t *)xsc;
    } else {
      q1.in = xs16;  // the token rows scaled once, staged by copy in every tile
      q1.in_scaled = 1;
      q1.in_rowsc = xsc;
    }
    q1.out_f32 = h32;
    q1.out_rowmax = hmax;
    q1.h_dbg = opts ? opts->h_out : nullptr;
    q1.row_list = ra.r.row_list;
    q1.bias = opts ? (const uint16_t *)opts->fc1_bias : nullptr;
    q1.relu = desc->activation == QMOE_ACT_RELU;
    set_swiglu(q1, opts);
    q1.act_dtype = desc->act_dtype;
    e = begin();
    if (e == hipSuccess) e = launch_grouped(q1, kGEpiSwiGLU, p.max_tiles, s);
    if (e == hipSuccess) e = end();
    if (e != hipSuccess) return hip_status(e, "grouped fc1");
    GroupedArgs q2 = grouped_base(L.fc2, pk + L.fc2_off, wsc + desc->num_experts);
    q2.tile_rows = p.tile_rows;
    q2.tile_info = ra.r.tile_info;
    q2.in = h32;
    q2.in_f32 = 1;
    q2.in_row_elems = desc->inter;
    q2.in_rowmax = hmax;
    q2.out_f32 = o;
    q2.bias = opts ? (const uint16_t *)opts->fc2_bias : nullptr;
    q2.act_dtype = desc->act_dtype;
    // a non-affine FC2 reads h split once into its scaled f16 parts (in
    // place), which every column tile then copies into LDS as they are
    const bool split_h = !L.fc2.affine;
    if (split_h) {
      q2.in_f32 = 0;
      q2.in_split = 1;
      q2.in_row_elems = 2 * (int64_t)desc->inter;  // halves per row
    }
    if (split_h) {
      e = begin();
      if (e == hipSuccess) e = launch_split_rows(h32, T * top_k, desc->inter, hmax, s);
      if (e == hipSuccess) e = end();
      if (e != hipSuccess) return hip_status(e, "split h");
    }
    e = begin();
    if (e == hipSuccess) e = launch_grouped(q2, kGEpiStoreF32, p.max_tiles, s);
    if (e == hipSuccess) e = end();
    if (e != hipSuccess) return hip_status(e, "grouped fc2");
    e = begin();
    if (e == hipSuccess)
      e = launch_combine(o, ra.r.slot_pos, ra.r.w, T, top_k, desc->hidden, desc->act_dtype, (uint16_t *)y, s);
    if (e == hipSuccess) e = end();
    if (e != hipSuccess) return hip_status(e, "combine");
    return copy_diagnostics(desc, opts, ra.r, (int64_t)T * top_k, s);
  }
  uint16_t *h_hi = (uint16_t *)(wsb + W.h_hi), *h_lo = (uint16_t *)(wsb + W.h_lo);

  GemvArgs g1 = gemv_base(L.fc1, pk + L.fc1_off);
  if (fc1_routes) {
    g1.logits = logits;
    g1.route_T = T;
    g1.route_E = desc->num_experts;
    g1.route_k = top_k;
    g1.route_max_slots = p.max_active;
    g1.route_softmax_all = p.softmax_all ? 1 : 0;
    g1.route = ra.r;
  }
  g1.slot_info = ra.r.slot_info;
  g1.token_of = ra.r.token_of;
  g1.row_list = ra.r.row_list;
  g1.top_k = top_k;
  g1.in = (const uint32_t *)(f32 ? x_hi : x);
  g1.in_row_pairs = desc->hidden / 2;
  g1.in_part_stride = f32 ? (int64_t)(x_lo - x_hi) / 2 : 0;
  g1.in_gather_token = 1;
  g1.h_hi = h_hi;
  g1.h_lo = h_lo;
  g1.h_dbg = opts ? opts->h_out : nullptr;
  g1.bias = opts ? (const uint16_t *)opts->fc1_bias : nullptr;
  g1.relu = desc->activation == QMOE_ACT_RELU;
  set_swiglu(g1, opts);
  g1.act_dtype = desc->act_dtype;
  g1.h_by_slot = p.fc2_cat;  // the concatenated FC2 reads the token's h rows in slot order
  e = begin();
  if (e == hipSuccess)
    e = launch_gemv(g1, fc1_routes ? kEpiSwiGLURouted : kEpiSwiGLU, gemv_in_mode(desc->act_dtype), p.mmax1,
                    p.ks1, p.tn1, L.fc1.block, p.max_active, s);
  if (e == hipSuccess) e = end();
  if (e != hipSuccess) return hip_status(e, "gemv fc1");

  GemvArgs g2 = gemv_base(L.fc2, pk + L.fc2_off);
  g2.slot_info = ra.r.slot_info;
  g2.token_of = ra.r.token_of;
  g2.row_list = ra.r.row_list;
  g2.top_k = f32 ? 0 : top_k;  // 1: FC2 writes y itself (16-bit y only); otherwise o and the combine
  g2.in = (const uint32_t *)h_hi;
  g2.in_row_pairs = desc->inter / 2;
  g2.in_part_stride = (int64_t)(h_lo - h_hi) / 2;
  g2.in_gather_token = 0;
  g2.out_f32 = o;
  g2.out_act = (uint16_t *)y;
  g2.act_dtype = desc->act_dtype;
  g2.bias = opts ? (const uint16_t *)opts->fc2_bias : nullptr;
  g2.route_w = ra.r.w;
  g2.route = ra.r;
  g2.route_k = top_k;
  g2.cat_stage = p.cat_stage;
  e = begin();
  if (e == hipSuccess)
    e = p.fc2_cat ? launch_gemv(g2, kEpiDownCat, 0, 1, p.ks2, p.tn2, L.fc2.block, 1, s)
                  : launch_gemv(g2, kEpiDown, 0, p.mmax2, p.ks2, p.tn2, L.fc2.block, p.max_active, s);
  if (e == hipSuccess) e = end();
  if (e != hipSuccess) return hip_status(e, "gemv fc2");
  if ((top_k > 1 || f32) && !p.fc2_cat) {
    e = begin();
    if (e == hipSuccess) e = launch_combine(o, ra.r.slot_pos, ra.r.w, T, top_k, desc->hidden, desc->act_dtype, y, s);
    if (e == hipSuccess) e = end();
    if (e != hipSuccess) return hip_status(e, "combine");
  }

  return copy_diagnostics(desc, opts, ra.r, (int64_t)T * top_k, s);
}

qmoe_status qmoe_forward(const qmoe_layer_desc *desc, const void *packed, const void *x,
                         const float *logits, int32_t T, int32_t top_k, void *y, void *ws,
                         size_t ws_bytes, void *stream) {
  return qmoe_forward_ex(desc, packed, x, logits, T, top_k, y, ws, ws_bytes, stream, nullptr);
}

// ------------------------------------------------- no-allocation forward
// The workspace of qmoe_forward_noalloc: one fixed device array per GPU the
// library runs on, held until the process ends.  In host code `scratch` only
// names the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[QMOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

qmoe_status scratch_for_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(QMOE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return fail(QMOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  e != hipSuccess ? hipGetErrorString(e) : "null address");
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}
}  // namespace

qmoe_status qmoe_forward_noalloc(const qmoe_layer_desc *desc, const void *packed, const void *x,
                                 const float *logits, int32_t T, int32_t top_k, void *y, void *stream) {
  qmoe_plan plan;
  qmoe_status st = qmoe_forward_plan(desc, T, top_k, nullptr, &plan);
  if (st != QMOE_OK) return st;
  if (T == 0) return ok();
  if (plan.workspace_bytes > (int64_t)QMOE_NOALLOC_SCRATCH_BYTES)
    return fail(QMOE_ERR_WORKSPACE_TOO_SMALL,
                "qmoe_forward_noalloc: %d tokens need %lld workspace bytes, the fixed scratch holds %lld",
                T, (long long)plan.workspace_bytes, (long long)QMOE_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != QMOE_OK) return st;
  return qmoe_forward_ex(desc, packed, x, logits, T, top_k, y, ws, (size_t)QMOE_NOALLOC_SCRATCH_BYTES, stream,
                         nullptr);
}

// ------------------------------------------------------ gathered channels
namespace {
constexpr uint64_t kChanMagic = 0x31304843454f4d51ull;  // "QMOECH01"
constexpr int32_t kChanMaxList = 65536;

qmoe_status check_channel_layer(const qmoe_layer_desc *d) {
  qmoe_status st = check_layer(d, true);
  if (st != QMOE_OK) return st;
  if (d->activation != QMOE_ACT_SWIGLU)
    return fail(QMOE_ERR_UNSUPPORTED, "gathered channels: SWIGLU layers only");
  if (d->act_dtype != QMOE_DTYPE_BF16 && d->act_dtype != QMOE_DTYPE_F16)
    return fail(QMOE_ERR_UNSUPPORTED, "gathered channels: bf16 or f16 activations only");
  if (qtype_affine(d->fc1.qtype) || qtype_affine(d->fc2.qtype))
    return fail(QMOE_ERR_UNSUPPORTED, "gathered channels: symmetric formats only (sym_int4, sym_int2, ternary)");
  if ((d->fc1.qtype == QMOE_QTYPE_TERNARY_B3) != (d->fc2.qtype == QMOE_QTYPE_TERNARY_B3))
    return fail(QMOE_ERR_UNSUPPORTED, "gathered channels: base-3 rows need both matrices in TERNARY_B3");
  if (d->fc1.qtype == QMOE_QTYPE_TERNARY_B3 && d->hidden > kChanMaxHiddenB3)
    return fail(QMOE_ERR_UNSUPPORTED, "gathered channels: base-3 rows need hidden <= %d", kChanMaxHiddenB3);
  if (d->hidden % d->fc2.block != 0)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "gathered channels: hidden %d not a multiple of fc2 block %d",
                d->hidden, d->fc2.block);
  if (d->hidden > kChanMaxHidden)
    return fail(QMOE_ERR_UNSUPPORTED, "gathered channels: hidden %d > %d", d->hidden, kChanMaxHidden);
  const ChanLayout L = ChanLayout::make(*d);
  if ((int64_t)d->num_experts * d->inter * (L.dn_row_bytes / 4) > (int64_t)UINT32_MAX)
    return fail(QMOE_ERR_UNSUPPORTED, "gathered channels: down projection beyond 16 GiB");
  return ok();
}

struct ChanWs {
  int64_t partial, end;
  int groups;
  static ChanWs make(const qmoe_layer_desc &d, int64_t T, int k, int C) {
    ChanWs w;
    Carve c;
    w.groups = (int)(((int64_t)k * C + kChanGroupEntries - 1) / kChanGroupEntries);
    w.partial = c.take(T * w.groups * (int64_t)d.hidden * 4);
    w.end = c.off;
    return w;
  }
};
}  // namespace

qmoe_status qmoe_channel_prepacked_size(const qmoe_layer_desc *desc, size_t *bytes) {
  qmoe_status st = check_channel_layer(desc);
  if (st != QMOE_OK) return st;
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  *bytes = (size_t)ChanLayout::make(*desc).total;
  return ok();
}

qmoe_status qmoe_channel_prepack(const qmoe_layer_desc *desc, const void *fc1_codes, const void *fc1_scales,
                                 const void *down_codes, const void *down_scales, void *dst, size_t dst_bytes,
                                 void *stream) {
  qmoe_status st = check_channel_layer(desc);
  if (st != QMOE_OK) return st;
  if (!fc1_codes || !fc1_scales || !down_codes || !down_scales || !dst)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "null source or destination pointer");
  if (!aligned(dst, kAlign)) return fail(QMOE_ERR_INVALID_ARGUMENT, "dst must be 256-byte aligned");
  if (!aligned(fc1_scales, 2) || !aligned(down_scales, 2))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "scale arrays must be 2-byte aligned");
  const ChanLayout L = ChanLayout::make(*desc);
  if (dst_bytes < (size_t)L.total)
    return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "dst holds %zu bytes, %lld needed", dst_bytes, (long long)L.total);
  const int64_t E = desc->num_experts, H = desc->hidden, I = desc->inter;
  const int64_t fc1_bytes = E * 2 * I * L.fc1_row_bytes, fc1_sc = E * 2 * I * (H / desc->fc1.block) * 2;
  const int64_t dn_bytes = E * I * L.dn_row_bytes, dn_sc = E * I * (H / desc->fc2.block) * 2;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *d = (uint8_t *)dst;
  uint8_t header[kHeaderBytes];
  memset(header, 0, sizeof header);
  const uint64_t magic = kChanMagic;
  memcpy(header, &magic, 8);
  memcpy(header + 8, desc, sizeof(qmoe_layer_desc) < 112 ? sizeof(qmoe_layer_desc) : 112);
  hipError_t e = hipMemcpyAsync(d, header, kHeaderBytes, hipMemcpyHostToDevice, s);
  uint32_t *err = (uint32_t *)(d + kErrWordOff);
  if (L.b3) {  // block records with the scales inside, and the invalid-byte count
    if (e == hipSuccess)
      e = launch_pack_b3_records((const uint8_t *)fc1_codes, (const uint16_t *)fc1_scales, E * 2 * I, H,
                                 desc->fc1.block, d + L.fc1_off, err, s);
    if (e == hipSuccess)
      e = launch_pack_b3_records((const uint8_t *)down_codes, (const uint16_t *)down_scales, E * I, H,
                                 desc->fc2.block, d + L.dn_off, err, s);
    if (e != hipSuccess) return hip_status(e, "channel prepack base-3 records");
  }
  if (!L.b3) {
    if (e == hipSuccess) e = hipMemcpyAsync(d + L.fc1_off, fc1_codes, fc1_bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(d + L.fc1_sc_off, fc1_scales, fc1_sc, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(d + L.dn_off, down_codes, dn_bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(d + L.dn_sc_off, down_scales, dn_sc, hipMemcpyDeviceToDevice, s);
  }
  if (e != hipSuccess) return hip_status(e, "channel prepack copies");
  if (desc->fc1.qtype == QMOE_QTYPE_TERNARY) e = launch_count_invalid_ternary(d + L.fc1_off, fc1_bytes, err, s);
  if (e == hipSuccess && desc->fc2.qtype == QMOE_QTYPE_TERNARY)
    e = launch_count_invalid_ternary(d + L.dn_off, dn_bytes, err, s);
  if (e != hipSuccess) return hip_status(e, "channel prepack ternary check");
  uint32_t nbad = 0;
  e = hipMemcpyAsync(&nbad, err, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "channel prepack error word");
  if (nbad)
    return fail(QMOE_ERR_INVALID_ARGUMENT, L.b3 ? "%u base-3 bytes hold more digits than allowed"
                                              : "%u ternary fields hold the invalid value 3",
                nbad);
  return ok();
}

qmoe_status qmoe_channel_workspace_size(const qmoe_layer_desc *desc, int32_t T, int32_t top_k, int32_t C,
                                        size_t *bytes) {
  qmoe_status st = check_channel_layer(desc);
  if (st == QMOE_OK) st = check_tokens(desc, T, top_k);
  if (st != QMOE_OK) return st;
  if (C < 1 || C > kChanMaxList) return fail(QMOE_ERR_INVALID_ARGUMENT, "list length C %d outside [1, %d]", C,
                                             kChanMaxList);
  if ((int64_t)T * top_k * C > INT32_MAX) return fail(QMOE_ERR_INVALID_ARGUMENT, "T * top_k * C overflows int32");
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  *bytes = (size_t)ChanWs::make(*desc, T, top_k, C).end;
  return ok();
}

qmoe_status qmoe_forward_channels(const qmoe_layer_desc *desc, const void *packed, const void *x,
                                  const float *logits, int32_t T, int32_t top_k, const int32_t *channels,
                                  int32_t C, void *y, void *ws, size_t ws_bytes, void *stream) {
  size_t need = 0;
  qmoe_status st = qmoe_channel_workspace_size(desc, T, top_k, C, &need);
  if (st != QMOE_OK) return st;
  if (T == 0) return ok();
  if (!packed || !x || !logits || !channels || !y || !ws) return fail(QMOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(packed, kAlign) || !aligned(ws, kAlign))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "packed and ws must be 256-byte aligned");
  if (!aligned(x, 16) || !aligned(y, 2) || !aligned(logits, 4) || !aligned(channels, 4))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "x must be 16-byte aligned (y 2, logits and channels 4)");
  if (ws_bytes < need)
    return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
  const ChanWs W = ChanWs::make(*desc, T, top_k, C);
  const ChanLayout L = ChanLayout::make(*desc);
  const uint8_t *pk = (const uint8_t *)packed;
  ChanArgs a{};
  a.fc1 = pk + L.fc1_off;
  a.fc1_scales = pk + L.fc1_sc_off;
  a.fc1_row_bytes = L.fc1_row_bytes;
  a.fc1_bits = qtype_bits(desc->fc1.qtype);
  a.fc1_block = desc->fc1.block;
  a.fc1_sf16 = desc->fc1.scale_dtype == QMOE_DTYPE_F16;
  a.fc1_zp = qtype_zero_point(desc->fc1.qtype);
  a.dn = pk + L.dn_off;
  a.dn_scales = pk + L.dn_sc_off;
  a.dn_row_bytes = L.dn_row_bytes;
  a.dn_bits = qtype_bits(desc->fc2.qtype);
  a.dn_block = desc->fc2.block;
  a.dn_sf16 = desc->fc2.scale_dtype == QMOE_DTYPE_F16;
  a.dn_zp = qtype_zero_point(desc->fc2.qtype);
  a.b3 = L.b3 ? 1 : 0;
  a.T = T;
  a.E = desc->num_experts;
  a.k = top_k;
  a.C = C;
  a.I = desc->inter;
  a.H = desc->hidden;
  a.groups = W.groups;
  a.x = (const uint16_t *)x;
  a.x_f16 = desc->act_dtype == QMOE_DTYPE_F16;
  a.logits = logits;
  a.channels = channels;
  a.partial = (float *)ws;
  a.y = (uint16_t *)y;
  hipStream_t s = (hipStream_t)stream;
  return hip_status(launch_channels(a, s), "gathered channels");
}

qmoe_status qmoe_route_workspace_size(int32_t T, int32_t E, int32_t top_k, size_t *bytes) {
  if (E < 1 || E > kMaxExperts) return fail(QMOE_ERR_UNSUPPORTED, "E %d outside [1, 256]", E);
  if (T < 0 || top_k < 1 || top_k > E || top_k > kMaxTopK || (int64_t)T * top_k > INT32_MAX)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "bad T/top_k");
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  Carve c;
  *bytes = (size_t)RouteWs::make(c, (int64_t)T * top_k, E).end;
  return ok();
}

qmoe_status qmoe_route(int32_t T, int32_t E, int32_t top_k, const float *logits, int32_t *ids,
                       float *w, int32_t *counts, int32_t *offsets, int32_t *row_list, void *ws,
                       size_t ws_bytes, void *stream) {
  size_t need = 0;
  qmoe_status st = qmoe_route_workspace_size(T, E, top_k, &need);
  if (st != QMOE_OK) return st;
  if (T == 0) return ok();
  if (!logits || !ids || !w || !counts || !offsets || !row_list || !ws)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  if (!aligned(ws, kAlign)) return fail(QMOE_ERR_INVALID_ARGUMENT, "ws must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  Carve c;
  const RouteWs R = RouteWs::make(c, (int64_t)T * top_k, E);
  RouteArgs ra;
  ra.logits = logits;
  ra.T = T;
  ra.E = E;
  ra.k = top_k;
  ra.r = R.bind((uint8_t *)ws);
  ra.topk_in_expand = (T <= 16) ? 1 : 0;
  ra.max_slots = (int)std::min<int64_t>(E, (int64_t)T * top_k);
  ra.zero_buf = nullptr;
  ra.zero_len = 0;
  ra.tile_rows = 0;
  ra.max_tiles = 0;
  ra.softmax_all = 0;
  hipError_t e = launch_route(ra, s);
  if (e != hipSuccess) return hip_status(e, "route");
  const int64_t S = (int64_t)T * top_k;
  e = hipMemcpyAsync(ids, ra.r.ids, S * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(w, ra.r.w, S * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(counts, ra.r.counts, (size_t)E * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(offsets, ra.r.offsets, ((size_t)E + 1) * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(row_list, ra.r.row_list, S * 4, hipMemcpyDeviceToDevice, s);
  return hip_status(e, "route copies");
}

qmoe_status qmoe_unpack_codes(const qmoe_layer_desc *desc, const void *packed, int32_t which,
                              int8_t *codes_out, void *stream) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  if (which != 1 && which != 2) return fail(QMOE_ERR_INVALID_ARGUMENT, "which must be 1 or 2");
  if (!packed || !codes_out) return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  if (!aligned(packed, kAlign)) return fail(QMOE_ERR_INVALID_ARGUMENT, "packed must be 256-byte aligned");
  const MoeLayout L = MoeLayout::make(*desc);
  const MatLayout &M = which == 1 ? L.fc1 : L.fc2;
  const int64_t off = which == 1 ? L.fc1_off : L.fc2_off;
  return hip_status(launch_unpack_matrix(M, desc->num_experts, (const uint8_t *)packed + off, codes_out,
                                         (hipStream_t)stream),
                    "unpack");
}

// ---------------------------------------------------------------- dense
qmoe_status qmoe_linear_prepacked_size(const qmoe_qmatrix_desc *desc, size_t *bytes) {
  if (!desc) return fail(QMOE_ERR_INVALID_ARGUMENT, "null descriptor");
  qmoe_status st = check_matrix(*desc, "linear", -1, -1);
  if (st == QMOE_OK && desc->qtype == QMOE_QTYPE_TERNARY_B3)
    st = fail(QMOE_ERR_UNSUPPORTED, "base-3 ternary rows are read by the gathered-channel calls only");
  if (st != QMOE_OK) return st;
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  *bytes = (size_t)(MatLayout::make(*desc).stride + kLinearTail);  // + the tail (error word, pre-scale)
  return ok();
}

qmoe_status qmoe_linear_prepack(const qmoe_qmatrix_desc *desc, const void *codes, const void *scales,
                                const void *biases, void *dst, size_t dst_bytes, void *stream) {
  size_t need = 0;
  qmoe_status st = qmoe_linear_prepacked_size(desc, &need);
  if (st != QMOE_OK) return st;
  const MatLayout L = MatLayout::make(*desc);
  if (!codes || !scales || !dst) return fail(QMOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (L.affine != (biases != nullptr))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "biases are required for affine formats and only for them");
  if (!aligned(dst, kAlign)) return fail(QMOE_ERR_INVALID_ARGUMENT, "dst must be 256-byte aligned");
  if (dst_bytes < need)
    return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "dst holds %zu bytes, %zu needed", dst_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  // The linear buffer has no header; invalid fields are counted in a word of
  // the 256-byte tail after the matrix.
  uint32_t *err = (uint32_t *)((uint8_t *)dst + L.stride);
  hipError_t e = hipMemsetAsync(err, 0, 4, s);
  if (e == hipSuccess)
    e = launch_prepack_matrix(L, 1, (const uint8_t *)codes, (const uint16_t *)scales,
                              (const uint16_t *)biases, (uint8_t *)dst, err, s);
  if (e == hipSuccess)
    e = launch_wscale(L, 1, (const uint8_t *)dst, (float *)((uint8_t *)dst + L.stride + kLinearWscOff), s);
  uint32_t nbad = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&nbad, err, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "linear prepack");
  if (nbad) return fail(QMOE_ERR_INVALID_ARGUMENT, "%u ternary fields hold the invalid value 3", nbad);
  return ok();
}

qmoe_status qmoe_linear_workspace_size(const qmoe_qmatrix_desc *desc, int32_t M, size_t *bytes) {
  size_t need = 0;
  qmoe_status st = qmoe_linear_prepacked_size(desc, &need);
  if (st != QMOE_OK) return st;
  if (M < 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "M must be >= 0");
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  *bytes = (size_t)align_up((int64_t)M * 4, kAlign);  // MFMA path: per-row activation scales
  return ok();
}

qmoe_status qmoe_linear(const qmoe_qmatrix_desc *desc, const void *packed, const void *x,
                        int32_t x_dtype, int32_t M, void *y, void *ws, size_t ws_bytes, int32_t path,
                        void *stream) {
  if (!desc) return fail(QMOE_ERR_INVALID_ARGUMENT, "null descriptor");
  qmoe_status st = check_matrix(*desc, "linear", -1, -1);
  if (st == QMOE_OK && desc->qtype == QMOE_QTYPE_TERNARY_B3)
    st = fail(QMOE_ERR_UNSUPPORTED, "base-3 ternary rows are read by the gathered-channel calls only");
  if (st != QMOE_OK) return st;
  if (x_dtype != QMOE_DTYPE_BF16 && x_dtype != QMOE_DTYPE_F16)
    return fail(QMOE_ERR_UNSUPPORTED, "x dtype %d not supported", x_dtype);
  if (M < 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "M must be >= 0");
  if (M == 0) return ok();
  if (path != QMOE_PATH_AUTO && path != QMOE_PATH_GEMV && path != QMOE_PATH_GROUPED)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "unknown path %d", path);
  const int pth = path == QMOE_PATH_AUTO ? (M <= kGemvMaxRowsDense ? QMOE_PATH_GEMV : QMOE_PATH_GROUPED) : path;
  if (pth == QMOE_PATH_GEMV && M > kGemvMaxRowsDense)
    return fail(QMOE_ERR_UNSUPPORTED, "GEMV path needs M <= %d", kGemvMaxRowsDense);
  if (!packed || !x || !y) return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  if (!aligned(packed, kAlign) || !aligned(x, 16) || !aligned(y, 16))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const MatLayout L = MatLayout::make(*desc);
  hipStream_t s = (hipStream_t)stream;
  if (pth == QMOE_PATH_GROUPED) {
    if (L.affine && L.nblk > kGroupedMaxAffineBlocks)
      return fail(QMOE_ERR_UNSUPPORTED, "affine formats on the MFMA path need K/block <= %d",
                  kGroupedMaxAffineBlocks);
    const size_t need = (size_t)align_up((int64_t)M * 4, kAlign);
    if (!ws) return fail(QMOE_ERR_INVALID_ARGUMENT, "the MFMA path needs a workspace");
    if (!aligned(ws, kAlign)) return fail(QMOE_ERR_INVALID_ARGUMENT, "ws must be 256-byte aligned");
    if (ws_bytes < need)
      return fail(QMOE_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
    float *xsc = (float *)ws;
    hipError_t e = launch_rowscale(x, M, L.K, x_dtype == QMOE_DTYPE_F16, xsc, nullptr, s);
    if (e != hipSuccess) return hip_status(e, "rowscale");
    GroupedArgs g = grouped_base(L, (const uint8_t *)packed,
                                 (const float *)((const uint8_t *)packed + L.stride + kLinearWscOff));
    g.dense_M = M;
    g.tile_rows = grouped_tile_rows(L.affine);
    g.in = x;
    g.in_f16 = x_dtype == QMOE_DTYPE_F16;
    g.in_row_elems = L.K;
    g.in_rowsc = xsc;
    g.out_act = (uint16_t *)y;
    g.act_dtype = x_dtype;
    return hip_status(launch_grouped(g, kGEpiStoreAct, (M + g.tile_rows - 1) / g.tile_rows, s), "linear mfma");
  }
  const GemvShape gs = pick_gemv(L.RG, L, M, kEpiStoreAct, x_dtype == QMOE_DTYPE_F16);
  GemvArgs g = gemv_base(L, (const uint8_t *)packed);
  g.dense_M = M;
  g.in = (const uint32_t *)x;
  g.in_row_pairs = L.K / 2;
  g.out_act = (uint16_t *)y;
  g.act_dtype = x_dtype;
  return hip_status(launch_gemv(g, kEpiStoreAct, x_dtype == QMOE_DTYPE_F16, M, gs.waves, gs.tn, L.block, 1, s),
                    "linear gemv");
}

qmoe_status qmoe_linear_unpack_codes(const qmoe_qmatrix_desc *desc, const void *packed,
                                     int8_t *codes_out, void *stream) {
  if (!desc) return fail(QMOE_ERR_INVALID_ARGUMENT, "null descriptor");
  qmoe_status st = check_matrix(*desc, "linear", -1, -1);
  if (st == QMOE_OK && desc->qtype == QMOE_QTYPE_TERNARY_B3)
    st = fail(QMOE_ERR_UNSUPPORTED, "base-3 ternary rows are read by the gathered-channel calls only");
  if (st != QMOE_OK) return st;
  if (!packed || !codes_out) return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  const MatLayout L = MatLayout::make(*desc);
  return hip_status(launch_unpack_matrix(L, 1, (const uint8_t *)packed, codes_out, (hipStream_t)stream),
                    "linear unpack");
}

// ---------------------------------------------------------- diagnostics
qmoe_status qmoe_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  if (!aligned(src, 16) || bytes % 16 != 0)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "src must be 16-byte aligned and bytes a multiple of 16");
  return hip_status(launch_read_probe(src, (int64_t)bytes, sink, device_cus(), (hipStream_t)stream), "read probe");
}

}  // extern "C"
