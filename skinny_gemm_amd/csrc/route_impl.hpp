// route_impl.hpp -- device-side routing used by the routing kernels and by
// the FC1 GEMV that routes small decode batches itself.
//
// The onnxruntime pull request 33005 (Description) reuses routing and
// expert-map kernels and expands the rows by expert before FC1.  Here:
//   top-k   one wavefront per token: lanes hold the logits, k rounds of a
//           wave-wide arg-max (ties to the lower expert index) select the
//           experts in descending order; weights = softmax of the selected
//           logits in fp32 (sum 1, exactly 1.0 for k = 1).
//   expand  (at most 64 slots) one wavefront, one slot per lane: a slot's
//           position in the expert-sorted list is the number of slots with
//           a smaller expert id plus its rank among the slots of its own
//           expert (lower slot index first), both counted from 8 ballots over
//           the expert id bits, most significant first.
#pragma once

#include <float.h>

#include "qmoe_internal.h"

namespace qmoe {

// Wave-wide top-k of one token.  Lane 0 writes the ids and weights to
// ids_out / w_out (when not null) and the ids to ids_lds (when not null).
__device__ inline void wave_topk(const float *__restrict__ l, int E, int k, int32_t *ids_out,
                                 float *w_out, int32_t *ids_lds) {
  const int lane = threadIdx.x & (kLanes - 1);
  float v[kMaxExperts / kLanes];
  bool taken[kMaxExperts / kLanes];
#pragma unroll
  for (int i = 0; i < kMaxExperts / kLanes; ++i) {
    const int e = lane + kLanes * i;
    v[i] = (e < E) ? l[e] : -FLT_MAX;
    taken[i] = (e >= E);
  }
  float sel_v[kMaxTopK];
  int sel_i[kMaxTopK];
  for (int j = 0; j < k; ++j) {
    float bv = -FLT_MAX;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxExperts / kLanes; ++i) {
      const int e = lane + kLanes * i;
      if (!taken[i] && (bi == 0x7FFFFFFF || v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxExperts / kLanes; ++i)
      if (lane + kLanes * i == bi) taken[i] = true;
    sel_v[j] = bv;
    sel_i[j] = bi;
  }
  if (lane == 0) {
    const float m = sel_v[0];
    float ex[kMaxTopK];
    float sum = 0.f;
    for (int j = 0; j < k; ++j) {
      ex[j] = expf(sel_v[j] - m);
      sum += ex[j];
    }
    for (int j = 0; j < k; ++j) {
      if (ids_out) ids_out[j] = sel_i[j];
      if (w_out) w_out[j] = ex[j] / sum;
      if (ids_lds) ids_lds[j] = sel_i[j];
    }
  }
}

// Expert map of S <= 64 slots by one wavefront.  ids: expert of each flat
// slot r = t*k + j (LDS); s_cnt: LDS scratch of kMaxExperts ints.  With r
// non-null the global lists are written (row_list, slot_pos, token_of,
// counts, offsets, active, num_active and max_slots entries of slot_info).
// With want >= 0, *slot_out (LDS) receives {expert, rows, first position, 0}
// of active expert number `want` (zero rows past the active experts) and
// slots_out[0..rows) (LDS) the flat slots of its rows in order (token =
// slot / k).
__device__ inline void wave_expand_small(const int32_t *ids, int S, int k, int E, int max_slots, int *s_cnt,
                                         const RouteBufs *r, int want, int4 *slot_out, int32_t *slots_out) {
  const int lane = threadIdx.x & (kLanes - 1);
  const bool valid = lane < S;
  const int e = valid ? ids[lane] : 0;
  uint64_t eq = __ballot(valid);
  int less = 0;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    const uint64_t ones = __ballot(valid && ((e >> b) & 1));
    if ((e >> b) & 1) {
      less += __popcll(eq & ~ones);  // same higher bits, 0 here: smaller id
      eq &= ones;
    } else {
      eq &= ~ones;
    }
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kLanes - lane));
  const int pos = less + __popcll(eq & below);
  // per-expert counts (LDS operations of one wavefront complete in order)
  for (int x = lane; x < kMaxExperts; x += kLanes) s_cnt[x] = 0;
  if (valid && (eq & below) == 0) s_cnt[e] = __popcll(eq);
  if (r && valid) {
    r->row_list[pos] = lane;
    r->slot_pos[lane] = pos;
    r->token_of[pos] = lane / k;
  }
  if (want >= 0 && lane == 0) *slot_out = make_int4(0, 0, 0, 0);
  // other lanes' LDS writes are read below: no reordering or forwarding
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();

  // exclusive scan of the counts and the active list
  constexpr int PER = kMaxExperts / kLanes;
  int c[PER], f[PER];
  int cs = 0, fs = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int x = lane * PER + i;
    c[i] = (x < E) ? s_cnt[x] : 0;
    f[i] = (c[i] > 0) ? 1 : 0;
    cs += c[i];
    fs += f[i];
  }
  int ci = cs, fi = fs;
#pragma unroll
  for (int off = 1; off < kLanes; off <<= 1) {
    const int oc = __shfl_up(ci, off), of = __shfl_up(fi, off);
    if (lane >= off) {
      ci += oc;
      fi += of;
    }
  }
  int run = ci - cs, frun = fi - fs;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int x = lane * PER + i;
    if (x < E) {
      if (r) {
        r->offsets[x] = run;
        r->counts[x] = c[i];
      }
      if (f[i]) {
        if (r) r->active[frun] = x;
        if (r && frun < max_slots) r->slot_info[frun] = make_int4(x, c[i], run, 0);
        if (frun == want) *slot_out = make_int4(x, c[i], run, 0);
      }
    }
    run += c[i];
    frun += f[i];
  }
  if (r) {
    if (lane == kLanes - 1) {
      r->offsets[E] = ci;
      r->num_active[0] = fi;
    }
    const int na = __shfl(fi, kLanes - 1);
    for (int sl = na + lane; sl < max_slots; sl += kLanes) r->slot_info[sl] = make_int4(0, 0, 0, 0);
  }
  if (want >= 0) {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const volatile int *sv = reinterpret_cast<const volatile int *>(slot_out);  // written above by one lane
    const int4 so = make_int4(sv[0], sv[1], sv[2], sv[3]);
    if (valid && so.y > 0 && e == so.x) slots_out[pos - so.z] = lane;
  }
}

}  // namespace qmoe
