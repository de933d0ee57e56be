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
#include <string.h>

#include <algorithm>
#include <string>

#include "qmoe_internal.h"

using namespace qmoe;

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
  if (m.qtype < QMOE_QTYPE_SYM_INT4 || m.qtype > QMOE_QTYPE_AFFINE_INT4)
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

qmoe_status check_layer(const qmoe_layer_desc *d) {
  if (!d) return fail(QMOE_ERR_INVALID_ARGUMENT, "null layer descriptor");
  if (d->num_experts < 1) return fail(QMOE_ERR_INVALID_ARGUMENT, "num_experts must be >= 1");
  if (d->num_experts > kMaxExperts)
    return fail(QMOE_ERR_UNSUPPORTED, "num_experts %d > %d", d->num_experts, kMaxExperts);
  if (d->hidden <= 0 || d->inter <= 0)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "hidden and inter must be positive");
  if (d->act_dtype != QMOE_DTYPE_BF16 && d->act_dtype != QMOE_DTYPE_F16)
    return fail(QMOE_ERR_UNSUPPORTED, "activation dtype %d not supported (bf16 or f16)", d->act_dtype);
  qmoe_status st = check_matrix(d->fc1, "fc1", 2 * (int64_t)d->inter, d->hidden);
  if (st != QMOE_OK) return st;
  return check_matrix(d->fc2, "fc2", d->hidden, d->inter);
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

struct RouteWs {
  int64_t ids, w, counts, offsets, row_list, slot_pos, active, num_active, end;
  static RouteWs make(Carve &c, int64_t S, int E) {
    RouteWs r;
    r.ids = c.take(S * 4);
    r.w = c.take(S * 4);
    r.counts = c.take((int64_t)E * 4);
    r.offsets = c.take(((int64_t)E + 1) * 4);
    r.row_list = c.take(S * 4);
    r.slot_pos = c.take(S * 4);
    r.active = c.take((int64_t)E * 4);
    r.num_active = c.take(4);
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
    b.active = (int32_t *)(ws + active);
    b.num_active = (int32_t *)(ws + num_active);
    return b;
  }
};

struct MoeWs {
  RouteWs route;
  int64_t h_hi, h_lo, o, total;
  static MoeWs make(const qmoe_layer_desc &d, int32_t T, int32_t k) {
    MoeWs w;
    Carve c;
    const int64_t S = (int64_t)T * k;
    w.route = RouteWs::make(c, S, d.num_experts);
    w.h_hi = c.take(S * d.inter * 2);
    w.h_lo = c.take(S * d.inter * 2);
    w.o = c.take(S * d.hidden * 4);
    w.total = c.off;
    return w;
  }
};

// ------------------------------------------------------------------ plan
constexpr size_t kLdsLimit = 64 * 1024;
constexpr int kTargetWaves = 2048;  // ~8 waves per CU on 256 CUs

int pick_mmax(int64_t rows) {
  int m = 1;
  while (m < rows && m < kGemvMaxRows) m <<= 1;
  return m;
}

// Waves per workgroup for the split-K GEMV: enough waves in flight to cover
// HBM latency, no more than the blocks along K, within the LDS budget.
int pick_waves(int64_t nwg, int64_t nblk, int mmax) {
  int64_t ks = (kTargetWaves + nwg - 1) / std::max<int64_t>(nwg, 1);
  ks = std::max<int64_t>(1, std::min<int64_t>(ks, 8));
  ks = std::min<int64_t>(ks, nblk);
  while (ks > 1 && gemv_lds_bytes(mmax, nblk, (int)ks) > kLdsLimit) --ks;
  if (gemv_lds_bytes(mmax, nblk, (int)ks) > kLdsLimit) return 0;
  return (int)ks;
}

struct Plan {
  int path;
  int mmax, ks1, ks2, max_active;
  int route_fused;
  int launches;
  std::string kernels;
};

qmoe_status make_plan(const qmoe_layer_desc &d, int32_t T, int32_t k, int path_req, Plan &p) {
  const MoeLayout L = MoeLayout::make(d);
  p = Plan{};
  int path = path_req;
  if (path == QMOE_PATH_AUTO) path = (T <= kGemvMaxRows) ? QMOE_PATH_GEMV : QMOE_PATH_GROUPED;
  if (path != QMOE_PATH_GEMV && path != QMOE_PATH_GROUPED)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "unknown path %d", path_req);
  if (path == QMOE_PATH_GEMV && T > kGemvMaxRows)
    return fail(QMOE_ERR_UNSUPPORTED, "GEMV path needs T <= %d (got %d)", kGemvMaxRows, T);
  if (path == QMOE_PATH_GROUPED)
    return fail(QMOE_ERR_UNSUPPORTED, "grouped MFMA path not available for T = %d", T);
  p.path = path;
  p.route_fused = (T <= 16) ? 1 : 0;
  p.max_active = (int)std::min<int64_t>(d.num_experts, (int64_t)T * k);
  p.mmax = pick_mmax(T);
  p.ks1 = pick_waves((int64_t)p.max_active * L.fc1.RG, L.fc1.nblk, p.mmax);
  p.ks2 = pick_waves((int64_t)p.max_active * L.fc2.RG, L.fc2.nblk, p.mmax);
  if (p.ks1 == 0 || p.ks2 == 0)
    return fail(QMOE_ERR_UNSUPPORTED, "K too large for the GEMV workgroup LDS budget");
  p.kernels = p.route_fused ? "route_expand" : "route_topk,route_expand";
  p.kernels += ",gemv_fc1_swiglu,gemv_fc2,combine";
  p.launches = p.route_fused ? 4 : 5;
  return ok();
}

qmoe_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(QMOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
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
  g.nblk = L.nblk;
  g.cpb = L.cpb;
  g.kc = L.kc;
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
  uint32_t nbad = 0;
  e = hipMemcpyAsync(&nbad, err, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "prepack error word");
  if (nbad) return fail(QMOE_ERR_INVALID_ARGUMENT, "%u ternary fields hold the invalid value 3", nbad);
  return ok();
}

qmoe_status qmoe_workspace_size(const qmoe_layer_desc *desc, int32_t T, int32_t top_k, size_t *bytes) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  st = check_tokens(desc, T, top_k);
  if (st != QMOE_OK) return st;
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  *bytes = (size_t)MoeWs::make(*desc, T, top_k).total;
  return ok();
}

qmoe_status qmoe_forward_plan(const qmoe_layer_desc *desc, int32_t T, int32_t top_k,
                              const qmoe_forward_opts *opts, qmoe_plan *plan) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  st = check_tokens(desc, T, top_k);
  if (st != QMOE_OK) return st;
  if (!plan) return fail(QMOE_ERR_INVALID_ARGUMENT, "null plan output");
  Plan p;
  st = make_plan(*desc, T, top_k, opts ? opts->path : QMOE_PATH_AUTO, p);
  if (st != QMOE_OK) return st;
  memset(plan, 0, sizeof *plan);
  plan->path = p.path;
  plan->num_launches = T == 0 ? 0 : p.launches;
  plan->gemv_mmax = p.mmax;
  plan->gemv_fc1_waves = p.ks1;
  plan->gemv_fc2_waves = p.ks2;
  plan->max_active = p.max_active;
  plan->workspace_bytes = MoeWs::make(*desc, T, top_k).total;
  snprintf(plan->kernels, sizeof plan->kernels, "%s", T == 0 ? "" : p.kernels.c_str());
  return ok();
}

qmoe_status qmoe_forward_ex(const qmoe_layer_desc *desc, const void *packed, const void *x,
                            const float *logits, int32_t T, int32_t top_k, void *y, void *ws,
                            size_t ws_bytes, void *stream, const qmoe_forward_opts *opts) {
  qmoe_status st = check_layer(desc);
  if (st != QMOE_OK) return st;
  st = check_tokens(desc, T, top_k);
  if (st != QMOE_OK) return st;
  if (opts && opts->reserved != 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "opts.reserved must be 0");
  if (T == 0) return ok();
  Plan p;
  st = make_plan(*desc, T, top_k, opts ? opts->path : QMOE_PATH_AUTO, p);
  if (st != QMOE_OK) return st;
  if (!packed || !x || !logits || !y || !ws)
    return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  if (!aligned(packed, kAlign) || !aligned(ws, kAlign))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "packed and ws must be 256-byte aligned");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(logits, 16))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "x, y and logits must be 16-byte aligned");
  const MoeWs W = MoeWs::make(*desc, T, top_k);
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
  hipError_t e = launch_route(ra, s);
  if (e != hipSuccess) return hip_status(e, "route");

  uint16_t *h_hi = (uint16_t *)(wsb + W.h_hi), *h_lo = (uint16_t *)(wsb + W.h_lo);
  float *o = (float *)(wsb + W.o);

  GemvArgs g1 = gemv_base(L.fc1, pk + L.fc1_off);
  g1.active = ra.r.active;
  g1.num_active = ra.r.num_active;
  g1.counts = ra.r.counts;
  g1.offsets = ra.r.offsets;
  g1.row_list = ra.r.row_list;
  g1.top_k = top_k;
  g1.in = (const uint32_t *)x;
  g1.in_row_pairs = desc->hidden / 2;
  g1.in_parts = 1;
  g1.in_gather_token = 1;
  g1.h_hi = h_hi;
  g1.h_lo = h_lo;
  g1.h_dbg = opts ? opts->h_out : nullptr;
  e = launch_gemv(g1, kEpiSwiGLU, desc->act_dtype == QMOE_DTYPE_F16, p.mmax, p.ks1, p.max_active, s);
  if (e != hipSuccess) return hip_status(e, "gemv fc1");

  GemvArgs g2 = gemv_base(L.fc2, pk + L.fc2_off);
  g2.active = ra.r.active;
  g2.num_active = ra.r.num_active;
  g2.counts = ra.r.counts;
  g2.offsets = ra.r.offsets;
  g2.row_list = ra.r.row_list;
  g2.top_k = top_k;
  g2.in = (const uint32_t *)h_hi;
  g2.in_row_pairs = desc->inter / 2;
  g2.in_parts = 2;
  g2.in_part_stride = (int64_t)(h_lo - h_hi) / 2;
  g2.in_gather_token = 0;
  g2.out_f32 = o;
  e = launch_gemv(g2, kEpiStoreF32, 0, p.mmax, p.ks2, p.max_active, s);
  if (e != hipSuccess) return hip_status(e, "gemv fc2");

  e = launch_combine(o, ra.r.slot_pos, ra.r.w, T, top_k, desc->hidden, desc->act_dtype, (uint16_t *)y, s);
  if (e != hipSuccess) return hip_status(e, "combine");

  const int64_t S = (int64_t)T * top_k;
  if (opts && opts->ids_out) {
    e = hipMemcpyAsync(opts->ids_out, ra.r.ids, S * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e, "ids copy");
  }
  if (opts && opts->w_out) {
    e = hipMemcpyAsync(opts->w_out, ra.r.w, S * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e, "weights copy");
  }
  if (opts && opts->counts_out) {
    e = hipMemcpyAsync(opts->counts_out, ra.r.counts, (size_t)desc->num_experts * 4,
                       hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e, "counts copy");
  }
  return ok();
}

qmoe_status qmoe_forward(const qmoe_layer_desc *desc, const void *packed, const void *x,
                         const float *logits, int32_t T, int32_t top_k, void *y, void *ws,
                         size_t ws_bytes, void *stream) {
  return qmoe_forward_ex(desc, packed, x, logits, T, top_k, y, ws, ws_bytes, stream, nullptr);
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
  if (st != QMOE_OK) return st;
  if (!bytes) return fail(QMOE_ERR_INVALID_ARGUMENT, "null size output");
  *bytes = (size_t)(MatLayout::make(*desc).stride + kAlign);  // + a tail for the prepack error word
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
  *bytes = 0;  // the GEMV path needs no workspace
  return ok();
}

qmoe_status qmoe_linear(const qmoe_qmatrix_desc *desc, const void *packed, const void *x,
                        int32_t x_dtype, int32_t M, void *y, void *ws, size_t ws_bytes, int32_t path,
                        void *stream) {
  (void)ws;
  (void)ws_bytes;
  if (!desc) return fail(QMOE_ERR_INVALID_ARGUMENT, "null descriptor");
  qmoe_status st = check_matrix(*desc, "linear", -1, -1);
  if (st != QMOE_OK) return st;
  if (x_dtype != QMOE_DTYPE_BF16 && x_dtype != QMOE_DTYPE_F16)
    return fail(QMOE_ERR_UNSUPPORTED, "x dtype %d not supported", x_dtype);
  if (M < 0) return fail(QMOE_ERR_INVALID_ARGUMENT, "M must be >= 0");
  if (M == 0) return ok();
  int pth = path == QMOE_PATH_AUTO ? QMOE_PATH_GEMV : path;
  if (pth != QMOE_PATH_GEMV) return fail(QMOE_ERR_UNSUPPORTED, "linear path %d not available", path);
  if (M > kGemvMaxRows) return fail(QMOE_ERR_UNSUPPORTED, "GEMV path needs M <= %d", kGemvMaxRows);
  if (!packed || !x || !y) return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  if (!aligned(packed, kAlign) || !aligned(x, 16) || !aligned(y, 16))
    return fail(QMOE_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const MatLayout L = MatLayout::make(*desc);
  const int mmax = pick_mmax(M);
  const int ks = pick_waves(L.RG, L.nblk, mmax);
  if (ks == 0) return fail(QMOE_ERR_UNSUPPORTED, "K too large for the GEMV workgroup LDS budget");
  GemvArgs g = gemv_base(L, (const uint8_t *)packed);
  g.dense_M = M;
  g.in = (const uint32_t *)x;
  g.in_row_pairs = L.K / 2;
  g.in_parts = 1;
  g.out_act = (uint16_t *)y;
  g.act_dtype = x_dtype;
  return hip_status(launch_gemv(g, kEpiStoreAct, x_dtype == QMOE_DTYPE_F16, mmax, ks, 1,
                                (hipStream_t)stream),
                    "linear gemv");
}

qmoe_status qmoe_linear_unpack_codes(const qmoe_qmatrix_desc *desc, const void *packed,
                                     int8_t *codes_out, void *stream) {
  if (!desc) return fail(QMOE_ERR_INVALID_ARGUMENT, "null descriptor");
  qmoe_status st = check_matrix(*desc, "linear", -1, -1);
  if (st != QMOE_OK) return st;
  if (!packed || !codes_out) return fail(QMOE_ERR_INVALID_ARGUMENT, "null device pointer");
  const MatLayout L = MatLayout::make(*desc);
  return hip_status(launch_unpack_matrix(L, 1, (const uint8_t *)packed, codes_out, (hipStream_t)stream),
                    "linear unpack");
}

}  // extern "C"
