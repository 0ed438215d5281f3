// dispatch.hip -- groups the T*k routed rows by expert.
//
// DS4Server issue #112, "Current upstream route" (sort_rows) and "Kernel
// contract": the routed slots are ordered by their expert id (a stable
// sort), with the inverse permutation and the token of every sorted row kept
// beside it, so the expert kernels can read x rows where they lie; the same
// section asks for per-expert row and tile prefix tables.  The PRD "5.5 real
// sparse MoE kernels (Metal)", "Acceptance criteria", names this step as the
// difficult one of the layer.
//
// A counting sort, stable and deterministic, in one workgroup:
//   1. each wave owns a contiguous segment of slots and counts its experts
//      with integer LDS atomics (order-independent);
//   2. block scans give expert offsets, and every (wave, expert) pair gets the
//      first position of its run: expert offset + counts of earlier waves;
//   3. each wave walks its segment in slot order, 64 slots at a time; lanes
//      that carry the same expert find each other with ballots over the bits
//      of the expert id, so a slot's rank = base + number of earlier equal
//      lanes, which is exactly the stable order.
// The same kernel emits the work plan the expert kernels consume: the list of
// experts with rows (plus the shared experts) and the list of row tiles.
#include <algorithm>

#include "device_common.h"
#include "dispatch_tiny.h"
#include "launch.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int kBatch = 8;   // slots per lane loaded together (long segments)
constexpr int kCache = 48;  // slots per lane kept in registers (segments up to 3072)
// Up to this many slots the whole dispatch runs in one workgroup; above it,
// in workgroups of dispatch_segment(N) slots (at most 256 workgroups).
constexpr int kSingleBlockMax = 4096;
inline int64_t dispatch_segment(int64_t N) {
  const int64_t per = (N + 255) / 256;
  return std::max<int64_t>(1024, (per + 255) / 256 * 256);
}

// In-place exclusive scan of a[0..n) (LDS); returns the total to every thread.
__device__ int block_exscan(int32_t *a, int n, int32_t *wave_tot) {
  const int tid = threadIdx.x, nth = blockDim.x, lane = tid & 63, w = tid >> 6;
  const int nw = nth / 64;
  const int chunk = (n + nth - 1) / nth;
  const int b = min(n, tid * chunk), e = min(n, b + chunk);
  int s = 0;
  for (int i = b; i < e; ++i) s += a[i];
  const int v = wave_incl_scan(s);
  if (lane == 63) wave_tot[w] = v;
  __syncthreads();
  if (w == 0) {
    const int wt = lane < nw ? wave_tot[lane] : 0;
    const int iv = wave_incl_scan(wt);
    if (lane < nw) wave_tot[lane] = iv - wt;
    if (lane == nw - 1) wave_tot[nw] = iv;
  }
  __syncthreads();
  int run = wave_tot[w] + v - s;
  for (int i = b; i < e; ++i) {
    const int t = a[i];
    a[i] = run;
    run += t;
  }
  const int total = wave_tot[nw];
  __syncthreads();
  return total;
}

// Work plan from per-expert offsets/counts held in LDS.  act_flag and
// tile_cnt are LDS scratch of length E.
__device__ void emit_plan(const int32_t *off, const int32_t *cnt, int32_t *act_flag,
                          int32_t *tile_cnt, int32_t *wave_tot, int E, int S, int N, int T, int tr,
                          int32_t *counters, PlanItem *act_items, PlanItem *tiles) {
  __shared__ int32_t s_multi;  // tiles that belong to experts with two or more tiles
  const int tid = threadIdx.x, nth = blockDim.x;
  if (tid == 0) s_multi = 0;
  __syncthreads();
  int multi = 0;
  for (int e = tid; e < E; e += nth) {
    act_flag[e] = cnt[e] > 0;
    tile_cnt[e] = (cnt[e] + tr - 1) / tr;
    if (tile_cnt[e] >= 2) multi += tile_cnt[e];
  }
  if (multi) atomicAdd(&s_multi, multi);
  __syncthreads();
  const int n_act = block_exscan(act_flag, E, wave_tot);
  const int n_tiles = block_exscan(tile_cnt, E, wave_tot);
  for (int e = tid; e < E; e += nth) {
    const int c = cnt[e];
    if (c > 0) act_items[act_flag[e]] = PlanItem{e, off[e], c, 0};
    for (int j = 0; j * tr < c; ++j)
      tiles[tile_cnt[e] + j] = PlanItem{e, off[e] + j * tr, min(tr, c - j * tr), 0};
  }
  const int shared_tiles = (T + tr - 1) / tr;
  for (int q = tid; q < S * shared_tiles; q += nth) {
    const int s = q / shared_tiles, j = q % shared_tiles;
    tiles[n_tiles + q] = PlanItem{E + s, N + s * T + j * tr, min(tr, T - j * tr), 0};
  }
  for (int s = tid; s < S; s += nth) act_items[n_act + s] = PlanItem{E + s, N + s * T, T, 0};
  if (tid == 0) {
    counters[0] = n_act + S;
    counters[1] = n_tiles + S * shared_tiles;
    counters[2] = plan_multi_tile(s_multi + (shared_tiles >= 2 ? S * shared_tiles : 0), counters[1]);
  }
}

// One wave's segment [i0, i1) of the flat slots: its expert ids, read once
// and kept in registers when the segment fits (all loads in flight
// together), otherwise re-read kBatch per lane at a time by each pass.
struct Segment {
  int i0, i1;
  bool cached;
  int cache[kCache];
};

__device__ __forceinline__ void seg_load(const int32_t *__restrict__ f, int i0, int i1, Segment &sg) {
  const int lane = threadIdx.x & 63;
  sg.i0 = i0;
  sg.i1 = i1;
  sg.cached = (i1 - i0) <= 64 * kCache;
  if (sg.cached) {
#pragma unroll
    for (int u = 0; u < kCache; ++u) {
      const int i = i0 + u * 64 + lane;
      sg.cache[u] = i < i1 ? f[i] : 0;
    }
  }
}

// Adds the segment's expert counts into cnt[E] (LDS, integer atomics, so the
// result does not depend on their order); sets *bad for an id outside [0, E).
__device__ __forceinline__ void seg_count(const int32_t *__restrict__ f, const Segment &sg, int E, int32_t *cnt,
                                          int32_t *bad) {
  const int lane = threadIdx.x & 63;
  if (sg.cached) {
#pragma unroll
    for (int u = 0; u < kCache; ++u) {
      if (sg.i0 + u * 64 + lane >= sg.i1) continue;
      const int e = sg.cache[u];
      if (unsigned(e) < unsigned(E)) atomicAdd(&cnt[e], 1);
      else *bad = 1;
    }
    return;
  }
  for (int b0 = sg.i0; b0 < sg.i1; b0 += kBatch * 64) {
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = b0 + u * 64 + lane;
      ev[u] = i < sg.i1 ? f[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (b0 + u * 64 + lane >= sg.i1) continue;
      const int e = ev[u];
      if (unsigned(e) < unsigned(E)) atomicAdd(&cnt[e], 1);
      else *bad = 1;
    }
  }
}

// Stable positions of the segment's slots, given base[e] = the first position
// of this wave's run of expert e (LDS, advanced in place).  The wave walks
// its segment in slot order, 64 slots at a time; lanes that carry the same
// expert find each other with ballots over the bits of the expert id, and a
// slot's position = base + number of earlier equal lanes.
__device__ __forceinline__ void seg_rank(const int32_t *__restrict__ f, const Segment &sg, int K, int E,
                                         volatile int32_t *base, int32_t *__restrict__ order,
                                         int32_t *__restrict__ inv_order, int32_t *__restrict__ row_map) {
  const int lane = threadIdx.x & 63;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 1;
  const uint64_t lt_mask = lane ? (~0ull >> (64 - lane)) : 0ull;
  auto rank_step = [&](int i, bool valid, int e) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(valid && bit);
      peers &= bit ? bal : ~bal;
    }
    if (valid) {
      const int pos = base[e] + __popcll(peers & lt_mask);
      order[pos] = i;
      inv_order[i] = pos;
      row_map[pos] = i / K;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == 63 - __clzll(peers)) base[e] = base[e] + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  };
  if (sg.cached) {
#pragma unroll
    for (int u = 0; u < kCache; ++u) {
      if (sg.i0 + u * 64 >= sg.i1) break;
      const int i = sg.i0 + u * 64 + lane;
      rank_step(i, i < sg.i1, sg.cache[u]);
    }
    return;
  }
  for (int bb = sg.i0; bb < sg.i1; bb += kBatch * 64) {
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = bb + u * 64 + lane;
      ev[u] = i < sg.i1 ? f[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = bb + u * 64 + lane;
      rank_step(i, i < sg.i1, ev[u]);
    }
  }
}

// Out-of-range expert id: an empty, in-bounds result with expert_off[E] = -1.
__device__ void write_bad(int N, int E, int32_t *order, int32_t *inv_order, int32_t *row_map,
                          int32_t *expert_off, int32_t *tile_off, int32_t *counters) {
  const int tid = threadIdx.x, nth = blockDim.x;
  for (int i = tid; i < N; i += nth) order[i] = inv_order[i] = row_map[i] = -1;
  for (int e = tid; e <= E; e += nth) {
    expert_off[e] = e == E ? -1 : 0;
    tile_off[e] = 0;
  }
  if (tid == 0) counters[0] = counters[1] = counters[2] = 0;
}

// Whole dispatch in one workgroup (small N).
__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const int32_t *__restrict__ f, int N, int K, int E, int S, int T, int tile_rows, int tr,
    int32_t *__restrict__ order, int32_t *__restrict__ inv_order, int32_t *__restrict__ row_map,
    int32_t *__restrict__ expert_off, int32_t *__restrict__ tile_off, int32_t *counters,
    PlanItem *act_items, PlanItem *tiles) {
  extern __shared__ int32_t lds[];
  const int nw = blockDim.x / 64;
  int32_t *cnt = lds;                 // [nw][E] per-wave counts, then run bases
  int32_t *off = cnt + nw * E;        // [E] expert offsets
  int32_t *tot = off + E;             // [E] expert counts
  int32_t *utile = tot + E;           // [E] caller tile offsets
  int32_t *scr0 = utile + E;          // [E] plan scratch
  int32_t *scr1 = scr0 + E;           // [E] plan scratch
  __shared__ int32_t wave_tot[17];
  __shared__ int32_t bad;

  const int tid = threadIdx.x, nth = blockDim.x, w = tid >> 6;
  for (int q = tid; q < nw * E; q += nth) cnt[q] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();

  const int seg = (N + nw - 1) / nw;
  const int i0 = min(N, w * seg), i1 = min(N, i0 + seg);
  Segment sg;
  seg_load(f, i0, i1, sg);
  seg_count(f, sg, E, cnt + w * E, &bad);
  __syncthreads();
  if (bad) {
    write_bad(N, E, order, inv_order, row_map, expert_off, tile_off, counters);
    return;
  }

  for (int e = tid; e < E; e += nth) {
    int c = 0;
    for (int ww = 0; ww < nw; ++ww) c += cnt[ww * E + e];
    tot[e] = c;
    off[e] = c;
    utile[e] = (c + tile_rows - 1) / tile_rows;
  }
  __syncthreads();
  block_exscan(off, E, wave_tot);
  const int n_utiles = block_exscan(utile, E, wave_tot);
  for (int e = tid; e < E; e += nth) {
    int run = off[e];
    for (int ww = 0; ww < nw; ++ww) {
      const int c = cnt[ww * E + e];
      cnt[ww * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  seg_rank(f, sg, K, E, cnt + w * E, order, inv_order, row_map);

  for (int e = tid; e < E; e += nth) {
    expert_off[e] = off[e];
    tile_off[e] = utile[e];
  }
  if (tid == 0) {
    expert_off[E] = N;
    tile_off[E] = n_utiles;
  }
  __syncthreads();
  emit_plan(off, tot, scr0, scr1, wave_tot, E, S, N, T, tr, counters, act_items, tiles);
}

// ---- many workgroups (large N): count, scan, rank ----
// Workgroup b owns slots [b*seg, (b+1)*seg), cut into one contiguous part
// per wave, so slot order = (workgroup, wave, lane) order and the ranks stay
// stable.  blk[b][0..E) holds the workgroup's expert counts; blk[b][E] flags
// an out-of-range id.

constexpr int kMbThreads = 256;
constexpr int kMbWaves = kMbThreads / 64;

__device__ __forceinline__ void mb_segment(int N, int seg, int &i0, int &i1) {
  const int b0 = blockIdx.x * seg, b1 = min(N, b0 + seg);
  const int wseg = (b1 - b0 + kMbWaves - 1) / kMbWaves, w = threadIdx.x >> 6;
  i0 = min(b1, b0 + w * wseg);
  i1 = min(b1, i0 + wseg);
}

__global__ __launch_bounds__(kMbThreads) void dispatch_count_kernel(const int32_t *__restrict__ f, int N, int E,
                                                                    int seg, int32_t *__restrict__ blk) {
  extern __shared__ int32_t lds[];  // [kMbWaves][E]
  __shared__ int32_t bad;
  const int tid = threadIdx.x, w = tid >> 6;
  for (int q = tid; q < kMbWaves * E; q += kMbThreads) lds[q] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  int i0, i1;
  mb_segment(N, seg, i0, i1);
  Segment sg;
  seg_load(f, i0, i1, sg);
  seg_count(f, sg, E, lds + w * E, &bad);
  __syncthreads();
  int32_t *row = blk + int64_t(blockIdx.x) * (E + 1);
  for (int e = tid; e < E; e += kMbThreads) {
    int c = 0;
#pragma unroll
    for (int ww = 0; ww < kMbWaves; ++ww) c += lds[ww * E + e];
    row[e] = c;
  }
  if (tid == 0) row[E] = bad;
}

// Workgroups 0..B-1 rank their own segments; each forms what it needs from
// blk: per expert the total over all workgroups (whose exclusive scan gives
// the expert offsets) and the sum over earlier workgroups (the start of this
// workgroup's run).  Workgroup B ranks nothing: it writes expert_off,
// tile_off and the work plan, off the rankers' path.  EPT: experts per
// thread (E <= EPT * 256); every blk row a thread reads is in flight at once
// (up to 24 workgroups per round).
template <int EPT>
__global__ __launch_bounds__(kMbThreads) void dispatch_rank_kernel(
    const int32_t *__restrict__ f, int N, int K, int E, int S, int T, int seg, int B, int tile_rows, int tr,
    const int32_t *__restrict__ blk, int32_t *__restrict__ order, int32_t *__restrict__ inv_order,
    int32_t *__restrict__ row_map, int32_t *__restrict__ expert_off, int32_t *__restrict__ tile_off,
    int32_t *counters, PlanItem *act_items, PlanItem *tiles) {
  extern __shared__ int32_t lds[];
  int32_t *cw = lds;                  // [kMbWaves][E] wave counts, then wave run starts
  int32_t *off = cw + kMbWaves * E;   // [E] expert offsets
  int32_t *tot = off + E;             // [E] expert counts
  int32_t *utile = tot + E;           // [E] caller tile offsets
  int32_t *pre = utile + E;           // [E] rows of each expert in earlier workgroups; plan scratch later
  int32_t *scr1 = pre + E;            // [E] plan scratch
  __shared__ int32_t wave_tot[17];
  __shared__ int32_t bad;
  const int tid = threadIdx.x, w = tid >> 6, b = blockIdx.x;
  const bool planner = b == B;

  int i0 = 0, i1 = 0;
  if (!planner) mb_segment(N, seg, i0, i1);
  Segment sg;
  seg_load(f, i0, i1, sg);
  for (int q = tid; q < kMbWaves * E; q += kMbThreads) cw[q] = 0;
  if (tid == 0) bad = 0;
  // column sums of blk (clamped indices: repeats are loaded but not added)
  constexpr int kRows = 24;
  int ctot[EPT], cpre[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) ctot[i] = cpre[i] = 0;
  for (int b0 = 0; b0 < B; b0 += kRows) {
    int v[EPT][kRows];
#pragma unroll
    for (int i = 0; i < EPT; ++i)
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const int e = min(tid + i * kMbThreads, E - 1);
        v[i][u] = blk[int64_t(min(b0 + u, B - 1)) * (E + 1) + e];
      }
#pragma unroll
    for (int i = 0; i < EPT; ++i)
#pragma unroll
      for (int u = 0; u < kRows; ++u)
        if (b0 + u < B) {
          ctot[i] += v[i][u];
          if (b0 + u < b) cpre[i] += v[i][u];
        }
  }
  __syncthreads();
  for (int q = tid; q < B; q += kMbThreads)
    if (blk[int64_t(q) * (E + 1) + E]) bad = 1;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + i * kMbThreads;
    if (e < E) {
      tot[e] = off[e] = ctot[i];
      pre[e] = cpre[i];
      utile[e] = (ctot[i] + tile_rows - 1) / tile_rows;
    }
  }
  __syncthreads();
  if (bad) {
    // Out-of-range expert id: the -1 result (each ranker its own positions).
    if (planner) {
      for (int e = tid; e <= E; e += kMbThreads) {
        expert_off[e] = e == E ? -1 : 0;
        tile_off[e] = 0;
      }
      if (tid == 0) counters[0] = counters[1] = counters[2] = 0;
    } else {
      const int p0 = b * seg, p1 = min(N, p0 + seg);
      for (int i = p0 + tid; i < p1; i += kMbThreads) order[i] = inv_order[i] = row_map[i] = -1;
    }
    return;
  }
  block_exscan(off, E, wave_tot);
  if (planner) {
    const int n_utiles = block_exscan(utile, E, wave_tot);
    for (int e = tid; e < E; e += kMbThreads) {
      expert_off[e] = off[e];
      tile_off[e] = utile[e];
    }
    if (tid == 0) {
      expert_off[E] = N;
      tile_off[E] = n_utiles;
    }
    __syncthreads();
    emit_plan(off, tot, pre, scr1, wave_tot, E, S, N, T, tr, counters, act_items, tiles);
    return;
  }
  seg_count(f, sg, E, cw + w * E, &bad);
  __syncthreads();
  for (int e = tid; e < E; e += kMbThreads) {
    int run = off[e] + pre[e];
#pragma unroll
    for (int ww = 0; ww < kMbWaves; ++ww) {
      const int c = cw[ww * E + e];
      cw[ww * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  seg_rank(f, sg, K, E, cw + w * E, order, inv_order, row_map);
}

// At most 64*SPL slots: one wave does it all.
template <int SPL>
__global__ __launch_bounds__(kWave) void dispatch_tiny_kernel(
    const int32_t *__restrict__ f, int N, int K, int E, int S, int T, int tile_rows, int tr, int32_t *order,
    int32_t *inv_order, int32_t *row_map, int32_t *expert_off, int32_t *tile_off, int32_t *counters,
    PlanItem *act_items, PlanItem *tiles) {
  __shared__ int32_t cnt[kMaxExperts];
  tiny_dispatch<SPL>(f, N, K, E, S, T, tile_rows, tr, order, inv_order, row_map, expert_off, tile_off, counters,
                     act_items, tiles, cnt);
}

__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t *__restrict__ expert_off,
                                                        int N, int E, int S, int T, int tr,
                                                        int32_t *counters, PlanItem *act_items,
                                                        PlanItem *tiles) {
  extern __shared__ int32_t lds[];
  int32_t *off = lds, *cnt = off + E, *scr0 = cnt + E, *scr1 = scr0 + E;
  __shared__ int32_t wave_tot[17];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // Clamp caller offsets into [0, N] so that a bad table cannot send the
    // expert kernels outside the sorted rows.
    const int a = min(max(expert_off[e], 0), N);
    const int b = min(max(expert_off[e + 1], a), N);
    off[e] = a;
    cnt[e] = b - a;
  }
  __syncthreads();
  emit_plan(off, cnt, scr0, scr1, wave_tot, E, S, N, T, tr, counters, act_items, tiles);
}

}  // namespace

int64_t dispatch_segment_slots(const moe_layer_desc *d, int32_t T) {
  const int64_t N = int64_t(T) * d->top_k;
  return N <= kSingleBlockMax ? 0 : dispatch_segment(N);
}

int64_t dispatch_scratch_ints(const moe_layer_desc *d, int32_t T) {
  const int64_t N = int64_t(T) * d->top_k;
  if (N <= kSingleBlockMax) return 0;
  const int64_t seg = dispatch_segment(N);
  return ((N + seg - 1) / seg) * (d->n_experts + 1);
}

void launch_dispatch(const moe_layer_desc *d, int32_t T, const int32_t *idx, int32_t tile_rows,
                     int32_t *order, int32_t *inv_order, int32_t *row_map, int32_t *expert_off,
                     int32_t *tile_off, int32_t *counters, PlanItem *act_items, PlanItem *tiles,
                     int32_t *scratch, void *stream, StageMarker *mk, bool counts_ready) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int tr = plan_tile_rows(d, T);
  const int E = d->n_experts, N = T * d->top_k;
  if (N <= kTinyMaxN) {
    auto tiny = [&](auto kern) {
      launch(kern, dim3(1), dim3(kWave), 0, s, idx, N, d->top_k, E, d->n_shared, T, tile_rows, tr, order,
                         inv_order, row_map, expert_off, tile_off, counters, act_items, tiles);
    };
    if (N <= 2 * kWave) tiny(dispatch_tiny_kernel<2>);
    else if (N <= 4 * kWave) tiny(dispatch_tiny_kernel<4>);
    else tiny(dispatch_tiny_kernel<8>);
  } else if (N <= kSingleBlockMax) {
    const int nw = kThreads / 64;
    const size_t lds = size_t(nw * E + 5 * E) * sizeof(int32_t);
    launch(dispatch_kernel, dim3(1), dim3(kThreads), lds, s, idx, N, d->top_k, E, d->n_shared, T,
                       tile_rows, tr, order, inv_order, row_map, expert_off, tile_off, counters, act_items, tiles);
  } else {
    // Scattered writes of order and row_map are spread over many CUs.
    const int seg = int(dispatch_segment(N));
    const int B = (N + seg - 1) / seg;
    const size_t lds_w = size_t(kMbWaves) * E * sizeof(int32_t);
    if (!counts_ready) launch(dispatch_count_kernel, dim3(B), dim3(kMbThreads), lds_w, s, idx, N, E, seg, scratch);
    // B ranking workgroups and one planning workgroup
    auto rank = [&](auto kern) {
      launch(kern, dim3(B + 1), dim3(kMbThreads), lds_w + size_t(5 * E) * sizeof(int32_t), s, idx, N,
                         d->top_k, E, d->n_shared, T, seg, B, tile_rows, tr, scratch, order, inv_order, row_map,
                         expert_off, tile_off, counters, act_items, tiles);
    };
    if (E <= kMbThreads) rank(dispatch_rank_kernel<1>);
    else if (E <= 2 * kMbThreads) rank(dispatch_rank_kernel<2>);
    else rank(dispatch_rank_kernel<kMaxExperts / kMbThreads>);
  }
  if (mk) mk->mark("dispatch");
}

void launch_plan(const moe_layer_desc *d, int32_t T, const int32_t *expert_off, int32_t *counters,
                 PlanItem *act_items, PlanItem *tiles, void *stream) {
  const int E = d->n_experts;
  const int tr = plan_tile_rows(d, T);
  const size_t lds = size_t(4 * E) * sizeof(int32_t);
  launch(plan_kernel, dim3(1), dim3(kThreads), lds, static_cast<hipStream_t>(stream),
                     expert_off, T * d->top_k, E, d->n_shared, T, tr, counters, act_items, tiles);
}

}  // namespace moe
