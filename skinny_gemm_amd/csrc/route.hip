// route.hip -- top-k routing and the per-expert row map (route_impl.hpp
// holds the per-wavefront pieces).
//
//   top-k   one wavefront per token (wave_topk).
//   expand  a stable counting sort of the flat slots r = t*k + j by expert,
//           over kPlaceRanges contiguous slot ranges: one wave per range
//           counts its rows per expert (64 slots a step, ranks inside a step
//           from ballots over the expert id bits); one workgroup turns the
//           counts into offsets (exclusive scan), the active experts, the
//           slot and tile lists and each range's first position per expert;
//           one wave per range writes its slots into row_list and the
//           inverse maps, so the per-slot work and the scattered stores are
//           spread over many compute units.
//   expand (fewer than kPlaceMinSlots slots) one workgroup sorts the slots
//           on its own (and for T <= 16 routes the tokens itself first).
//   small   (T*k <= 64 slots, no tile list) one workgroup: one wavefront
//           per token for the top-k, then one wavefront builds every list
//           from ballots (wave_expand_lists).
#include "route_impl.hpp"

namespace qmoe {

constexpr int kExpandThreads = 1024;
constexpr int kExpandWaves = kExpandThreads / kLanes;

template <bool ALL>
__global__ __launch_bounds__(256) void route_topk_kernel(RouteArgs a) {
  __shared__ TopkScratch s_tk[256 / kLanes];
  const int t = blockIdx.x * (blockDim.x / kLanes) + (threadIdx.x / kLanes);
  if (t >= a.T) return;
  wave_topk<ALL>(a.logits + (int64_t)t * a.E, a.E, a.k, a.r.ids + (int64_t)t * a.k,
            a.r.w + (int64_t)t * a.k, nullptr, &s_tk[threadIdx.x / kLanes]);
}

constexpr int kSmallCachedTiles = 16;  // slot ids per thread held in registers by the one-workgroup expand

// Small batches: one workgroup (which with topk_in_expand, T <= kExpandWaves,
// first routes the tokens itself, one wave per token) builds the LDS histogram
// -> counts, the exclusive scan -> offsets, the active experts and the slot
// and tile lists, then sorts the slots stably by expert one tile of
// kExpandThreads slots at a time (rank inside a wave from ballots over the
// expert id bits, ranks across waves from per-wave counts in LDS).
template <bool ALL>
__global__ __launch_bounds__(kExpandThreads) void route_expand_one_kernel(RouteArgs a) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_wc[2][kExpandWaves][kMaxExperts];  // per tile parity: wave counts, then prefixes
  __shared__ int32_t s_ids[kExpandWaves * kMaxTopK];
  __shared__ TopkScratch s_tk[kExpandWaves];
  const int tid = threadIdx.x, lane = tid & (kLanes - 1), wave = tid / kLanes;
  const int E = a.E;
  const int S = a.T * a.k;
  const bool fused = a.topk_in_expand != 0;

  if (fused && wave < a.T) {
    wave_topk<ALL>(a.logits + (int64_t)wave * E, E, a.k, a.r.ids + (int64_t)wave * a.k,
              a.r.w + (int64_t)wave * a.k, s_ids + wave * a.k, &s_tk[wave]);
  }
  for (int e = tid; e < kMaxExperts; e += kExpandThreads) {
    s_cnt[e] = 0;
    s_base[e] = 0;
  }
  for (int i = tid; i < a.zero_len; i += kExpandThreads) a.zero_buf[i] = 0;
  for (int i = tid; i < 2 * kExpandWaves * kMaxExperts; i += kExpandThreads) (&s_wc[0][0][0])[i] = 0;
  __syncthreads();

  // the first kSmallCachedTiles tiles of slot ids, loaded once into registers
  // (one memory latency for all of them instead of one per tile)
  int ecache[kSmallCachedTiles];
#pragma unroll
  for (int i = 0; i < kSmallCachedTiles; ++i) {
    const int r = i * kExpandThreads + tid;
    ecache[i] = (r < S) ? (fused ? s_ids[r] : a.r.ids[r]) : 0;
  }
#pragma unroll
  for (int i = 0; i < kSmallCachedTiles; ++i)
    if (i * kExpandThreads + tid < S) atomicAdd(&s_cnt[ecache[i]], 1);
  for (int r = kSmallCachedTiles * kExpandThreads + tid; r < S; r += kExpandThreads) {
    const int e = fused ? s_ids[r] : a.r.ids[r];
    atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();

  // Exclusive scan of counts and compaction of the active experts (wave 0).
  if (wave == 0) {
    constexpr int PER = kMaxExperts / kLanes;
    int c[PER], f[PER];
    int cs = 0, fs = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      c[i] = (e < E) ? s_cnt[e] : 0;
      f[i] = (c[i] > 0) ? 1 : 0;
      cs += c[i];
      fs += f[i];
    }
    int ci = cs, fi = fs;  // inclusive scans across lanes
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
      const int e = lane * PER + i;
      if (e < E) {
        s_off[e] = run;
        a.r.offsets[e] = run;
        a.r.counts[e] = c[i];
        if (f[i]) {
          a.r.active[frun] = e;
          if (frun < a.max_slots) a.r.slot_info[frun] = make_int4(e, c[i], run, 0);
        }
      }
      run += c[i];
      frun += f[i];
    }
    if (lane == kLanes - 1) {
      s_off[E] = ci;
      a.r.offsets[E] = ci;
      a.r.num_active[0] = fi;
    }
    // slots past the active experts do no work
    const int na = __shfl(fi, kLanes - 1);
    for (int sl = na + lane; sl < a.max_slots; sl += kLanes) a.r.slot_info[sl] = make_int4(0, 0, 0, 0);

    // grouped path: tiles of tile_rows rows per expert, in expert order; every
    // entry's last field holds the number of tiles (the grouped kernels map
    // their workgroups over that many)
    if (a.tile_rows > 0) {
      int nt[PER];
      int ts = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        nt[i] = (c[i] + a.tile_rows - 1) / a.tile_rows;
        ts += nt[i];
      }
      int ti = ts;
#pragma unroll
      for (int off = 1; off < kLanes; off <<= 1) {
        const int o = __shfl_up(ti, off);
        if (lane >= off) ti += o;
      }
      int tpos = ti - ts;
      int roff = ci - cs;
      const int ntot = __shfl(ti, kLanes - 1);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = lane * PER + i;
        for (int t = 0; t < nt[i]; ++t)
          if (tpos + t < a.max_tiles)
            a.r.tile_info[tpos + t] =
                make_int4(e, roff + t * a.tile_rows, min(a.tile_rows, c[i] - t * a.tile_rows), ntot);
        tpos += nt[i];
        roff += c[i];
      }
      for (int t = ntot + lane; t < a.max_tiles; t += kLanes) a.r.tile_info[t] = make_int4(0, 0, 0, ntot);
    }
  }
  __syncthreads();

  // Stable scatter, one tile of kExpandThreads slots at a time (ids of the
  // first tiles from registers, later ones loaded).
  auto scatter = [&](int t0, int e) __attribute__((always_inline)) {
    const int r = t0 + tid;
    const bool valid = r < S;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bb = __ballot(valid && ((e >> b) & 1));
      same &= ((e >> b) & 1) ? bb : ~bb;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kLanes - lane));
    const int rank = __popcll(same & below);
    const int pb = (t0 / kExpandThreads) & 1;  // this tile's buffer (all zero on entry)
    if (valid && rank == 0) s_wc[pb][wave][e] = __popcll(same);
    __syncthreads();
    // per expert: the wave counts become exclusive prefixes over the waves
    // (plus the rows of earlier tiles), the base moves past this tile, and
    // the other buffer -- read by the previous tile before the barrier
    // above -- is cleared for the next tile
    for (int x = tid; x < E; x += kExpandThreads) {
      int run = s_base[x];
      for (int w2 = 0; w2 < kExpandWaves; ++w2) {
        const int c = s_wc[pb][w2][x];
        s_wc[pb][w2][x] = run;
        s_wc[pb ^ 1][w2][x] = 0;
        run += c;
      }
      s_base[x] = run;
    }
    __syncthreads();
    if (valid) {
      const int pos = s_off[e] + s_wc[pb][wave][e] + rank;
      a.r.row_list[pos] = r;
      a.r.slot_pos[r] = pos;
      a.r.token_of[pos] = r / a.k;
    }
  };
#pragma unroll
  for (int i = 0; i < kSmallCachedTiles; ++i)
    if (i * kExpandThreads < S) scatter(i * kExpandThreads, ecache[i]);
  for (int t0 = kSmallCachedTiles * kExpandThreads; t0 < S; t0 += kExpandThreads) {
    const int r = t0 + tid;
    scatter(t0, r < S ? (fused ? s_ids[r] : a.r.ids[r]) : 0);
  }
}

// Slot ranges: kPlaceRanges contiguous ranges of whole 64-slot steps.
__device__ inline int place_range_steps(int S) {
  const int steps_all = (S + kLanes - 1) / kLanes;
  return (steps_all + kPlaceRanges - 1) / kPlaceRanges;
}

// Lanes of a 64-slot step holding expert e (valid lanes only; expert ids
// < 256, 8 id bits) and this lane's rank among them; rank 0 leads.
__device__ inline void step_match(bool valid, int e, uint64_t &same, int &rank) {
  const int lane = threadIdx.x & (kLanes - 1);
  same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t bb = __ballot(valid && ((e >> b) & 1));
    same &= ((e >> b) & 1) ? bb : ~bb;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kLanes - lane));
  rank = __popcll(same & below);
}

// Single workgroup, after route_topk_kernel and route_count_kernel: from
// the rows of each expert in each slot range, the counts, offsets, the
// active experts, the slot and tile lists and each range's first position
// per expert; route_place_kernel then writes the row list.
template <bool ALL>
__global__ __launch_bounds__(kExpandThreads) void route_expand_kernel(RouteArgs a) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_rc[kPlaceRanges][kMaxExperts];  // per range: count, then exclusive prefix over ranges
  __shared__ int s_seg[kExpandThreads / kMaxExperts][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & (kLanes - 1), wave = tid / kLanes;
  const int E = a.E;
  for (int i = tid; i < a.zero_len; i += kExpandThreads) a.zero_buf[i] = 0;
  for (int i = tid; i < kPlaceRanges * kMaxExperts; i += kExpandThreads) {
    const int q = i / kMaxExperts, e = i % kMaxExperts;
    s_rc[q][e] = e < E ? a.r.range_base[q * E + e] : 0;
  }
  __syncthreads();
  // Per expert: segment sums of 16 ranges, then each range's count becomes
  // the exclusive prefix over the earlier ranges, and the total the count.
  constexpr int kSegs = kExpandThreads / kMaxExperts, kPerSeg = kPlaceRanges / kSegs;
  const int ex = tid % kMaxExperts, seg = tid / kMaxExperts;
  {
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPerSeg; ++i) sum += s_rc[seg * kPerSeg + i][ex];
    s_seg[seg][ex] = sum;
  }
  __syncthreads();
  {
    int run = 0;
#pragma unroll
    for (int j = 0; j < kSegs; ++j) run += j < seg ? s_seg[j][ex] : 0;
#pragma unroll
    for (int i = 0; i < kPerSeg; ++i) {
      const int c = s_rc[seg * kPerSeg + i][ex];
      s_rc[seg * kPerSeg + i][ex] = run;
      run += c;
    }
    if (seg == kSegs - 1) s_cnt[ex] = run;
  }
  __syncthreads();

  // Exclusive scan of counts and compaction of the active experts (wave 0).
  if (wave == 0) {
    constexpr int PER = kMaxExperts / kLanes;
    int c[PER], f[PER];
    int cs = 0, fs = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      c[i] = (e < E) ? s_cnt[e] : 0;
      f[i] = (c[i] > 0) ? 1 : 0;
      cs += c[i];
      fs += f[i];
    }
    int ci = cs, fi = fs;  // inclusive scans across lanes
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
      const int e = lane * PER + i;
      if (e < E) {
        s_off[e] = run;
        a.r.offsets[e] = run;
        a.r.counts[e] = c[i];
        if (f[i]) {
          a.r.active[frun] = e;
          if (frun < a.max_slots) a.r.slot_info[frun] = make_int4(e, c[i], run, 0);
        }
      }
      run += c[i];
      frun += f[i];
    }
    if (lane == kLanes - 1) {
      s_off[E] = ci;
      a.r.offsets[E] = ci;
      a.r.num_active[0] = fi;
    }
    // slots past the active experts do no work
    const int na = __shfl(fi, kLanes - 1);
    for (int sl = na + lane; sl < a.max_slots; sl += kLanes) a.r.slot_info[sl] = make_int4(0, 0, 0, 0);

    // grouped path: tiles of tile_rows rows per expert, in expert order; every
    // entry's last field holds the number of tiles (the grouped kernels map
    // their workgroups over that many)
    if (a.tile_rows > 0) {
      int nt[PER];
      int ts = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        nt[i] = (c[i] + a.tile_rows - 1) / a.tile_rows;
        ts += nt[i];
      }
      int ti = ts;
#pragma unroll
      for (int off = 1; off < kLanes; off <<= 1) {
        const int o = __shfl_up(ti, off);
        if (lane >= off) ti += o;
      }
      int tpos = ti - ts;
      int roff = ci - cs;
      const int ntot = __shfl(ti, kLanes - 1);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = lane * PER + i;
        for (int t = 0; t < nt[i]; ++t)
          if (tpos + t < a.max_tiles)
            a.r.tile_info[tpos + t] =
                make_int4(e, roff + t * a.tile_rows, min(a.tile_rows, c[i] - t * a.tile_rows), ntot);
        tpos += nt[i];
        roff += c[i];
      }
      for (int t = ntot + lane; t < a.max_tiles; t += kLanes) a.r.tile_info[t] = make_int4(0, 0, 0, ntot);
    }
  }
  __syncthreads();

  // each range's first position per expert, for the placing kernel
  for (int i = tid; i < kPlaceRanges * E; i += kExpandThreads) {
    const int q = i / E, e = i - q * E;
    a.r.range_base[i] = s_off[e] + s_rc[q][e];
  }
}

// One wave per slot range (after a top-k kernel): the range's rows of each
// expert, into range_base [range][expert] for the expand kernel.
__global__ __launch_bounds__(kLanes) void route_count_kernel(RouteArgs a) {
  __shared__ int s_c[kMaxExperts];
  const int lane = threadIdx.x;
  const int q = blockIdx.x, E = a.E, S = a.T * a.k;
  for (int e = lane; e < E; e += kLanes) s_c[e] = 0;
  __syncthreads();
  constexpr int kChunk = 8;
  const int spr = place_range_steps(S);
  for (int c0 = 0; c0 < spr; c0 += kChunk) {
    int ev[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int r = (q * spr + c0 + i) * kLanes + lane;
      ev[i] = (c0 + i < spr && r < S) ? a.r.ids[r] : 0;
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int r = (q * spr + c0 + i) * kLanes + lane;
      const bool valid = c0 + i < spr && r < S;
      uint64_t same;
      int rank;
      step_match(valid, ev[i], same, rank);
      if (valid && rank == 0) s_c[ev[i]] += __popcll(same);
    }
  }
  __syncthreads();
  for (int e = lane; e < E; e += kLanes) a.r.range_base[q * E + e] = s_c[e];
}

// One wave per slot range: the range's slots in order, each at its
// expert's next position (the range's first position per expert plus the
// rows placed so far, plus the rank inside the step).  Gives row_list, its
// inverse slot_pos and token_of.
__global__ __launch_bounds__(kLanes) void route_place_kernel(RouteArgs a) {
  __shared__ int s_run[kMaxExperts];
  const int lane = threadIdx.x;
  const int q = blockIdx.x, E = a.E, S = a.T * a.k;
  for (int e = lane; e < E; e += kLanes) s_run[e] = a.r.range_base[q * E + e];
  __syncthreads();
  constexpr int kChunk = 8;
  const int spr = place_range_steps(S);
  for (int c0 = 0; c0 < spr; c0 += kChunk) {
    int ev[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int r = (q * spr + c0 + i) * kLanes + lane;
      ev[i] = (c0 + i < spr && r < S) ? a.r.ids[r] : 0;
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int r = (q * spr + c0 + i) * kLanes + lane;
      const bool valid = c0 + i < spr && r < S;
      uint64_t same;
      int rank;
      step_match(valid, ev[i], same, rank);
      if (valid) {
        const int pos = s_run[ev[i]] + rank;
        a.r.row_list[pos] = r;
        a.r.slot_pos[r] = pos;
        a.r.token_of[pos] = r / a.k;
      }
      // every lane has read the entry before its leader moves it on (one
      // wave: the read above executes before this write)
      if (valid && rank == 0) s_run[ev[i]] += __popcll(same);
    }
  }
}

// Small decode batches (T * k <= 64 slots, no grouped-path lists): one wave
// per token routes it, then wave 0 alone builds the expert map.
template <bool ALL>
__global__ __launch_bounds__(1024) void route_small_kernel(RouteArgs a) {
  __shared__ int32_t s_ids[kExpandWaves * kMaxTopK];
  __shared__ TopkScratch s_tk[kExpandWaves];
  const int wave = threadIdx.x / kLanes;
  if (wave < a.T)
    wave_topk<ALL>(a.logits + (int64_t)wave * a.E, a.E, a.k, a.r.ids + (int64_t)wave * a.k,
              a.r.w + (int64_t)wave * a.k, s_ids + wave * a.k, &s_tk[wave]);
  __syncthreads();
  if (wave == 0) wave_expand_lists(s_ids, a.T * a.k, a.k, a.E, a.max_slots, a.r);
}

// The ALL instances (unnormalised top-k weights) only when the call asks for them.
template <bool ALL>
hipError_t launch_route_as(const RouteArgs &a, hipStream_t s) {
  if (a.topk_in_expand && a.T > 0 && (int64_t)a.T * a.k <= kLanes && a.tile_rows == 0 && a.zero_len == 0)
    return qlaunch(route_small_kernel<ALL>, dim3(1), dim3(a.T * kLanes), 0, s, a);
  // many slots: counted and placed one wave per slot range around the
  // expand workgroup; fewer: the one-workgroup sort (three fewer launches)
  const bool ranged = !a.topk_in_expand && (int64_t)a.T * a.k >= kPlaceMinSlots;
  if (!a.topk_in_expand && a.T > 0) {
    const int per = 256 / kLanes;
    hipError_t e = qlaunch(route_topk_kernel<ALL>, dim3((a.T + per - 1) / per), dim3(256), 0, s, a);
    if (e == hipSuccess && ranged) e = qlaunch(route_count_kernel, dim3(kPlaceRanges), dim3(kLanes), 0, s, a);
    if (e != hipSuccess) return e;
  }
  if (!ranged) return qlaunch(route_expand_one_kernel<ALL>, dim3(1), dim3(kExpandThreads), 0, s, a);
  const hipError_t e = qlaunch(route_expand_kernel<ALL>, dim3(1), dim3(kExpandThreads), 0, s, a);
  if (e != hipSuccess) return e;
  return qlaunch(route_place_kernel, dim3(kPlaceRanges), dim3(kLanes), 0, s, a);
}

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
  return a.softmax_all ? launch_route_as<true>(a, s) : launch_route_as<false>(a, s);
}

}  // namespace qmoe
