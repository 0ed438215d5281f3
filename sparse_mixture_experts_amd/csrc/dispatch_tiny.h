// dispatch_tiny.h -- the dispatch of a handful of routed rows in one wave.
//
// The same outputs as the workgroup dispatch (DS4Server issue #112, "Current
// upstream route": order, inv_order, row_map; "Kernel contract": per-expert
// row and tile prefix tables; plus the internal work plan) for N <= 64*SPL
// flat slots (SPL slots per lane, at most 8), computed by a single wave so
// that no workgroup barrier or second kernel is needed: used by the dispatch
// entry point for small N and by the router's selection kernel when every
// token of the call is in one workgroup (decode).
#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kTinyMaxN = 8 * kWave;        // the dispatch entry point's one-wave path
constexpr int kTinyFusedMaxN = 2 * kWave;   // dispatch inside the router's selection kernel

// f: the N expert ids (flat slot i = t*K + j), global or LDS.  cnt: LDS
// scratch of E ints owned by this wave.  tile_rows: the caller's tile_off
// granularity; tr: the row-tile height of the internal plan.
template <int SPL>
__device__ __forceinline__ void tiny_dispatch(const int32_t *f, int N, int K, int E, int S, int T, int tile_rows,
                                              int tr, int32_t *order, int32_t *inv_order, int32_t *row_map,
                                              int32_t *expert_off, int32_t *tile_off, int32_t *counters,
                                              PlanItem *act_items, PlanItem *tiles, int32_t *cnt) {
  const int lane = lane_id();
  int ev[SPL];  // expert of slot h*64 + lane
  bool bad = false;
#pragma unroll
  for (int h = 0; h < SPL; ++h) {
    const int i = h * kWave + lane;
    ev[h] = i < N ? f[i] : 0;
    bad |= i < N && unsigned(ev[h]) >= unsigned(E);
  }
  if (__ballot(bad)) {
    // Out-of-range expert id: an empty, in-bounds result with expert_off[E] = -1.
    for (int i = lane; i < N; i += kWave) order[i] = inv_order[i] = row_map[i] = -1;
    for (int e = lane; e <= E; e += kWave) {
      expert_off[e] = e == E ? -1 : 0;
      tile_off[e] = 0;
    }
    if (lane == 0) counters[0] = counters[1] = counters[2] = 0;
    return;
  }
  for (int e = lane; e < E; e += kWave) cnt[e] = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < SPL; ++h)
    if (h * kWave + lane < N) atomicAdd(&cnt[ev[h]], 1);
  __builtin_amdgcn_wave_barrier();

  // Each lane owns a contiguous run of experts; exclusive scans of the rows,
  // caller tiles, plan tiles and active experts of the runs.
  const int chunk = (E + kWave - 1) / kWave;
  const int b = min(E, lane * chunk), b1 = min(E, b + chunk);
  int rs = 0, us = 0, ps = 0, as = 0, ms = 0;
  for (int e = b; e < b1; ++e) {
    const int c = cnt[e];
    rs += c;
    us += (c + tile_rows - 1) / tile_rows;
    ps += (c + tr - 1) / tr;
    as += c > 0;
    if (c > tr) ms += (c + tr - 1) / tr;  // tiles of experts with two or more
  }
  const int multi = wave_incl_scan(ms);
  // inclusive scans
  const int rx = wave_incl_scan(rs), ux = wave_incl_scan(us), px = wave_incl_scan(ps), ax = wave_incl_scan(as);
  const int n_utiles = read_lane_i(ux, kWave - 1), n_ptiles = read_lane_i(px, kWave - 1);
  const int n_act = read_lane_i(ax, kWave - 1);
  int r = rx - rs, u = ux - us, pt = px - ps, ac = ax - as;  // exclusive bases of this lane's run
  for (int e = b; e < b1; ++e) {
    const int c = cnt[e];
    expert_off[e] = r;
    tile_off[e] = u;
    if (c > 0) {
      act_items[ac++] = PlanItem{e, r, c, 0};
      for (int j = 0; j * tr < c; ++j) tiles[pt++] = PlanItem{e, r + j * tr, min(tr, c - j * tr), 0};
    }
    cnt[e] = r;  // run start of expert e, advanced by the ranking below
    r += c;
    u += (c + tile_rows - 1) / tile_rows;
  }
  const int shared_tiles = (T + tr - 1) / tr;
  for (int q = lane; q < S * shared_tiles; q += kWave) {
    const int s = q / shared_tiles, j = q % shared_tiles;
    tiles[n_ptiles + q] = PlanItem{E + s, N + s * T + j * tr, min(tr, T - j * tr), 0};
  }
  for (int s = lane; s < S; s += kWave) act_items[n_act + s] = PlanItem{E + s, N + s * T, T, 0};
  if (lane == 0) {
    expert_off[E] = N;
    tile_off[E] = n_utiles;
    counters[0] = n_act + S;
    counters[1] = n_ptiles + S * shared_tiles;
    counters[2] = plan_multi_tile(read_lane_i(multi, kWave - 1) + (shared_tiles >= 2 ? S * shared_tiles : 0),
                                  counters[1]);
  }
  __builtin_amdgcn_wave_barrier();

  // Stable positions, 64 slots at a time: lanes with the same expert find each
  // other with ballots over the bits of the id.
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 1;
  const uint64_t lt_mask = lane ? (~0ull >> (kWave - lane)) : 0ull;
  volatile int32_t *base = cnt;
#pragma unroll
  for (int h = 0; h < SPL; ++h) {
    const int i = h * kWave + lane;
    const bool valid = i < N;
    const int e = ev[h];
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bal = __ballot(valid && on);
      peers &= on ? bal : ~bal;
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
  }
}

}  // namespace moe
