// route_impl.hpp -- device-side routing used by the routing kernels and by
// the FC1 GEMV that routes small decode batches itself.
//
// The onnxruntime pull request 33005 (Description) reuses routing and
// expert-map kernels and expands the rows by expert before FC1.  Here:
//   top-k   one wavefront per token selects the experts in descending
//           logit order (ties to the lower expert index) in k rounds, each
//           a DPP wave maximum over the experts not yet taken and the lowest
//           expert holding it; weights = softmax of the selected logits in
//           fp32 (sum 1, exactly 1.0 for k = 1).
//   expand  (at most 64 slots) one wavefront, one slot per lane: a slot's
//           position in the expert-sorted list is the number of slots with
//           a smaller expert id plus its rank among the slots of its own
//           expert (lower slot index first), both counted from 8 ballots over
//           the expert id bits, most significant first; an expert's rank
//           among the active experts comes from the same ballots over the
//           first slot of each expert.
#pragma once

#include <float.h>

#include "qmoe_internal.h"

namespace qmoe {

// Per-wave LDS scratch of wave_topk: the selected experts and logits in
// selection order.
struct TopkScratch {
  int32_t id[kMaxTopK];
  float v[kMaxTopK];
};

// Maximum of v over the wavefront, in every lane: DPP row shifts reduce
// each row of 16 lanes, row broadcasts combine the rows (lanes without a
// source keep -inf), lane 63 ends with the maximum and is read back.
__device__ inline float wave_max(float v) {
  constexpr int kRowShr = 0x110, kBcast15 = 0x142, kBcast31 = 0x143;
  const int ninf = __float_as_int(-__builtin_inff());
  float m = v;
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(m), kRowShr + 1, 0xf, 0xf, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(m), kRowShr + 2, 0xf, 0xf, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(m), kRowShr + 4, 0xf, 0xf, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(m), kRowShr + 8, 0xf, 0xf, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(m), kBcast15, 0xa, 0xf, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(m), kBcast31, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), kLanes - 1));
}

// Sum of v over the wavefront, in every lane (xor butterfly).
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < kLanes; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Wave-wide top-k of one token.  Lane 0 writes the ids and weights to
// ids_out / w_out (when not null) and the ids to ids_lds (when not null),
// in selection order.  Requires 1 <= k <= E.
//
// Selection order: an expert's position is the number of logits greater
// than its own plus the number of equal logits of lower index (the k rounds
// of first-strictly-greater arg-max, ties to the lower index, for finite
// logits).  Each of the k rounds takes a DPP wave maximum over the experts
// not yet taken and the lowest expert holding it (one logit per lane for
// E <= 64, E / 64 per lane beyond).  The selection is recorded in sc; the
// weights are computed by lane 0 in fp32 in selection order: the softmax of
// the selected logits, or (ALL) exp(l - max) over the wave sum of
// exp(l - max) of all E logits, the selected entries of the softmax over
// every expert.
template <bool ALL = false>
__device__ inline void wave_topk(const float *__restrict__ l, int E, int k, int32_t *ids_out, float *w_out,
                                 int32_t *ids_lds, TopkScratch *sc) {
  const int lane = threadIdx.x & (kLanes - 1);
  float all_sum = 0.f;  // ALL: sum of exp(l - max) over all E logits
  // the selection goes to sc->id / sc->v in selection order (LDS: no
  // private arrays indexed by the runtime k)
  if (E <= kLanes) {
    // k rounds of arg-max: the wave maximum of the experts not yet taken
    // (DPP), then the lowest lane holding it
    const bool have = lane < E;
    const float v = have ? l[lane] : -__builtin_inff();
    bool avail = have;
    for (int j = 0; j < k; ++j) {
      const float m = wave_max(avail ? v : -__builtin_inff());
      const uint64_t at = __ballot(avail && v == m);
      const int sel = at ? __builtin_ctzll(at) : 0;
      if (lane == sel) avail = false;
      if (lane == 0) {
        sc->id[j] = sel;
        sc->v[j] = m;
      }
      if constexpr (ALL) {
        if (j == 0) all_sum = wave_sum(have ? expf(v - m) : 0.f);
      }
    }
  } else {
    // the same rounds over E / 64 logits per lane (expert lane + 64 i):
    // the lane maximum, the wave maximum, then the lowest expert holding it
    constexpr int PER = kMaxExperts / kLanes;
    float v[PER];
    unsigned avail = 0;  // bit i: expert lane + 64 i present and not taken
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + kLanes * i;
      v[i] = (e < E) ? l[e] : -__builtin_inff();
      avail |= (e < E) ? (1u << i) : 0u;
    }
    for (int j = 0; j < k; ++j) {
      float lm = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < PER; ++i) lm = fmaxf(lm, ((avail >> i) & 1u) ? v[i] : -__builtin_inff());
      const float m = wave_max(lm);
      int sel = -1;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint64_t at = __ballot(((avail >> i) & 1u) && v[i] == m);
        if (sel < 0 && at) sel = kLanes * i + __builtin_ctzll(at);
      }
      if (sel < 0) sel = 0;
      if (lane == (sel & (kLanes - 1))) avail &= ~(1u << (sel / kLanes));
      if (lane == 0) {
        sc->id[j] = sel;
        sc->v[j] = m;
      }
      if constexpr (ALL) {
        if (j == 0) {
          float part = 0.f;
#pragma unroll
          for (int i = 0; i < PER; ++i) part += (lane + kLanes * i < E) ? expf(v[i] - m) : 0.f;
          all_sum = wave_sum(part);
        }
      }
    }
  }
  // lane 0 recorded the selection above and computes the weights
  if (lane == 0) {
    const float m = sc->v[0];
    float sum = all_sum;
    if constexpr (!ALL)
      for (int j = 0; j < k; ++j) sum += expf(sc->v[j] - m);
    for (int j = 0; j < k; ++j) {
      const int id = sc->id[j];
      if (ids_out) ids_out[j] = id;
      if (w_out) w_out[j] = expf(sc->v[j] - m) / sum;
      if (ids_lds) ids_lds[j] = id;
    }
  }
}

// The expert map entry of active expert number `want` alone, by one
// wavefront from ballots (no LDS histogram): *slot_out (LDS) receives
// {expert, rows, first position, 0} (zeros past the active experts) and
// slots_out[0..rows) (LDS) the flat slots of its rows in order.  Active
// experts are numbered in increasing id; a slot's position counts the
// slots of smaller id, then the slots of its own id with lower index, as
// in wave_expand_lists.
__device__ inline void wave_expand_want(const int32_t *ids, int S, int want, int4 *slot_out, int32_t *slots_out) {
  const int lane = threadIdx.x & (kLanes - 1);
  if (S == 1) {  // one slot: one active expert with one row
    if (lane == 0) {
      *slot_out = want == 0 ? make_int4(ids[0], 1, 0, 0) : make_int4(0, 0, 0, 0);
      if (want == 0) slots_out[0] = 0;
    }
    return;
  }
  const bool valid = lane < S;
  const int e = valid ? ids[lane] : 0;
  // slots of smaller id (less) and of the same id (eq)
  uint64_t eq = __ballot(valid);
  int less = 0;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    const uint64_t ones = __ballot(valid && ((e >> b) & 1));
    if ((e >> b) & 1) {
      less += __popcll(eq & ~ones);
      eq &= ones;
    } else {
      eq &= ~ones;
    }
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kLanes - lane));
  const int pos = less + __popcll(eq & below);
  // distinct smaller ids: the same count over the first slot of each id
  const bool first = valid && (eq & below) == 0;
  uint64_t feq = __ballot(first);
  int fless = 0;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    const uint64_t ones = __ballot(first && ((e >> b) & 1));
    if ((e >> b) & 1) {
      fless += __popcll(feq & ~ones);
      feq &= ones;
    } else {
      feq &= ~ones;
    }
  }
  const bool mine = valid && fless == want;
  const uint64_t found = __ballot(first && fless == want);
  if (found == 0ull) {
    if (lane == 0) *slot_out = make_int4(0, 0, 0, 0);
  } else {
    if (first && fless == want) *slot_out = make_int4(e, __popcll(eq), less, 0);
    if (mine) slots_out[pos - less] = lane;
  }
}

// The global expert map of S <= 64 slots by one wavefront, from ballots
// and a pass over the slot ids (no histogram scan): row_list, slot_pos,
// token_of, counts, offsets (E + 1), active, num_active and the max_slots
// entries of slot_info (zeros past the active experts).  ids: expert of
// each flat slot r = t*k + j (LDS).
__device__ inline void wave_expand_lists(const int32_t *ids, int S, int k, int E, int max_slots,
                                         const RouteBufs &r) {
  const int lane = threadIdx.x & (kLanes - 1);
  const bool valid = lane < S;
  const int e = valid ? ids[lane] : 0;
  uint64_t eq = __ballot(valid);
  int less = 0;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    const uint64_t ones = __ballot(valid && ((e >> b) & 1));
    if ((e >> b) & 1) {
      less += __popcll(eq & ~ones);
      eq &= ones;
    } else {
      eq &= ~ones;
    }
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kLanes - lane));
  const int pos = less + __popcll(eq & below);
  const bool first = valid && (eq & below) == 0;
  const uint64_t firsts = __ballot(first);
  uint64_t feq = firsts;
  int fless = 0;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    const uint64_t ones = __ballot(first && ((e >> b) & 1));
    if ((e >> b) & 1) {
      fless += __popcll(feq & ~ones);
      feq &= ones;
    } else {
      feq &= ~ones;
    }
  }
  const int na = __popcll(firsts);
  if (valid) {
    r.row_list[pos] = lane;
    r.slot_pos[lane] = pos;
    r.token_of[pos] = lane / k;
  }
  if (first) {
    r.active[fless] = e;
    if (fless < max_slots) r.slot_info[fless] = make_int4(e, __popcll(eq), less, 0);
  }
  for (int sl = na + lane; sl < max_slots; sl += kLanes) r.slot_info[sl] = make_int4(0, 0, 0, 0);
  // per expert: rows routed to it and rows of smaller id
  for (int x = lane; x < E; x += kLanes) {
    int c = 0, off = 0;
    for (int q = 0; q < S; ++q) {
      const int id = ids[q];
      c += id == x ? 1 : 0;
      off += id < x ? 1 : 0;
    }
    r.counts[x] = c;
    r.offsets[x] = off;
  }
  if (lane == 0) {
    r.offsets[E] = S;
    r.num_active[0] = na;
  }
}

}  // namespace qmoe
