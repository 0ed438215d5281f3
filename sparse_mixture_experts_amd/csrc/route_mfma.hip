// route_mfma.hip -- router for many tokens: matrix-core logits, certified by
// exact recomputation of the few experts that can still reach the top-k.
//
// The top-k experts and their order must equal those of the fixed fp32
// logit order (64-column chunks, each a sequential fma chain from +0, chunk
// partials added in ascending order, bias last).  Computing every logit that
// way costs 2*T*d*E fp32 fmas on the vector units.  Instead:
//   1. the router weight is transposed to [E][d] (its columns become
//      contiguous rows) and the per-expert squared norms are formed;
//   2. L~ = x . W + bias on the bf16 matrix cores (exact bf16 products, fp32
//      sums: two MFMAs per 64-column chunk from zero, chunk results added in
//      fp32).  fp16 layers split every value exactly into a bf16 head and a
//      bf16 tail (fp16's 11 significant bits fit in two bf16 parts, and
//      bf16's exponent range holds fp16's subnormals) and take all four
//      head/tail products, so L~ is again a sum of exact products;
//   3. per token, with B = gamma * ||x_t|| * max_e ||W_e|| + gamma * max|bias|
//      a bound on |L~ - L| for every expert (Cauchy-Schwarz bounds the sum of
//      |x_i W_ie|; gamma covers the rounding of both summation orders), every
//      expert whose true logit can reach the top-k satisfies L~ >= L~_(k) - 2B
//      (the k-th order statistic moves by at most B).  Only those candidates
//      are recomputed in the fixed order, and the top-k is chosen among them
//      exactly (larger logit first, lower index on ties).  When more than 64
//      experts are candidates (near-ties, e.g. x = 0), every expert of that
//      token is recomputed.
// Softmax weights use the recomputed logits of the selected experts; with
// renormalisation the all-expert denominator cancels, so L~ may stand in for
// the non-candidates there.  ("MoE Optimization COMPLETE", "Mega Kernel
// Architecture": router matmul, softmax and top-K all on the GPU.)
#include "device_common.h"
#include "f16_stage.h"
#include "launch.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// Eight fp16 values -> head and tail bf16 vectors with head + tail exact.
__device__ __forceinline__ void f16x8_split(uint4 v, bf16x8 &hd, bf16x8 &tl) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[4], t[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = f16_lo(u[p]), b = f16_hi(u[p]);
    h[p] = pack_bf16(a, b);
    t[p] = pack_bf16(a - bf16_lo(h[p]), b - bf16_hi(h[p]));
  }
  hd = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  tl = __builtin_bit_cast(bf16x8, make_uint4(t[0], t[1], t[2], t[3]));
}

constexpr int kThreads = 256;
constexpr int kChunk = 64;
constexpr int kMaxCand = 64;


// ---- 1. transpose W [d][E] -> WT [E][d] and squared-norm partials ---------
// Block (eb, kb): experts eb*64.., columns kb*256..; normp[kb][e] = sum of
// squares of W[kb*256 .. +256][e].
template <int DT>
__global__ __launch_bounds__(kThreads) void router_transpose_kernel(const uint16_t *__restrict__ w, int D, int E,
                                                                    uint16_t *__restrict__ wt,
                                                                    float *__restrict__ normp,
                                                                    int32_t *__restrict__ counts, int n_counts) {
  __shared__ uint16_t tile[64][256 + 8];
  const int tid = threadIdx.x;
  // the dispatch counts that the certification adds to start from zero
  for (int i = (blockIdx.y * gridDim.x + blockIdx.x) * kThreads + tid; i < n_counts;
       i += gridDim.x * gridDim.y * kThreads)
    counts[i] = 0;
  const int e0 = blockIdx.x * 64, k0 = blockIdx.y * 256;
  {
    const int k = k0 + tid;  // one router row per thread, 64 experts
    if (k < D && e0 + 64 <= E && E % 8 == 0) {
#pragma unroll
      for (int j8 = 0; j8 < 8; ++j8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(w + int64_t(k) * E + e0 + j8 * 8);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          tile[j8 * 8 + 2 * h][tid] = uint16_t(u[h] & 0xffffu);
          tile[j8 * 8 + 2 * h + 1][tid] = uint16_t(u[h] >> 16);
        }
      }
    } else {
      for (int j = 0; j < 64; ++j) {
        const int e = e0 + j;
        tile[j][tid] = (k < D && e < E) ? w[int64_t(k) * E + e] : uint16_t(0);
      }
    }
  }
  __syncthreads();
  const int el = tid / 4, q = tid % 4;  // expert row, quarter of the 256 columns
  const int e = e0 + el;
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint4 v = *reinterpret_cast<const uint4 *>(&tile[el][q * 64 + c * 8]);
    const float f[8] = {half_lo<DT>(v.x), half_hi<DT>(v.x), half_lo<DT>(v.y), half_hi<DT>(v.y),
                        half_lo<DT>(v.z), half_hi<DT>(v.z), half_lo<DT>(v.w), half_hi<DT>(v.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(f[i], f[i], ss);
    const int k = k0 + q * 64 + c * 8;
    if (e < E && k < D) *reinterpret_cast<uint4 *>(wt + int64_t(e) * D + k) = v;
  }
  ss += __shfl_xor(ss, 1, kWave);
  ss += __shfl_xor(ss, 2, kWave);
  if (q == 0 && e < E) normp[int64_t(blockIdx.y) * E + e] = ss;
}

// ---- 2. L~ = x . W + bias on MFMA ------------------------------------------
// Block tile 64 experts x 64 tokens, 8 waves; wave (we, wt) owns 32 experts x
// 16 tokens = 2 MFMA tiles.  The grid is (expert tiles, token tiles, runs):
// run z takes one of gridDim.z equal runs of the 64-column chunks and writes
// its own partial L~ (lt + z*T*E); the certification adds the partials in z
// order.  Operand A = WT rows (experts), operand B = x rows (tokens); a
// lane's 4 results are 4 consecutive experts of one token.
// The blocks of the first token tile also add up the squared-norm partials of
// their 64 experts: normp[n_kb][e] -> normp[n_kb + 0 * E + e] (the row after
// the partials).
constexpr int kMfThreads = 512;
template <int DT>
__global__ __launch_bounds__(kMfThreads) void router_mfma_kernel(const uint16_t *__restrict__ x,
                                                                 const uint16_t *__restrict__ wt,
                                                                 const float *__restrict__ bias,
                                                                 float *__restrict__ normp, int n_kb, int T,
                                                                 int D, int E, float *__restrict__ lt,
                                                                 int norms_ready, int32_t *__restrict__ counts,
                                                                 int n_counts) {
  __shared__ uint16_t sab[2][2][64][kChunk + 8];  // [buffer][expert tile, token tile][row][col]
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lr = lane & 15, lg = lane >> 4;
  // XCD-aware order.  Workgroups go to the 8 XCDs round-robin by linear id;
  // each XCD takes a contiguous range of (expert tile fastest, token tile,
  // chunk run) items, so the expert tiles of a token tile run on one XCD and
  // read that token tile through the same L2 (x is then fetched once, not
  // once per XCD).
  const int nbx = gridDim.x, nby = gridDim.y, total = nbx * nby * gridDim.z;
  const int lin = (blockIdx.z * nby + blockIdx.y) * nbx + blockIdx.x;
  const int item = total % 8 == 0 ? (lin % 8) * (total / 8) + lin / 8 : lin;
  const int bx = item % nbx, by = (item / nbx) % nby, bz = item / (nbx * nby);
  const int e0 = bx * 64, t0 = by * 64;
  // with a prepared router the transpose kernel does not run: its other
  // job, zeroing the dispatch counts that the certification adds to, is done
  // here
  for (int i = lin * kMfThreads + tid; i < n_counts; i += total * kMfThreads) counts[i] = 0;
  if (!norms_ready && by == 0 && bz == 0 && tid < 64 && e0 + tid < E) {
    float s = 0.f;
    for (int kb = 0; kb < n_kb; ++kb) s += normp[int64_t(kb) * E + e0 + tid];
    normp[int64_t(n_kb) * E + e0 + tid] = s;
  }
  const int we = wave / 4, wtk = wave % 4;
  f32x4 acc[2];
  acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // staging: threads 0..255 fill the expert tile, 256..511 the token tile;
  // thread -> (row (tid % 256) / 4, 16 columns (tid % 4) * 16).  kRing chunks
  // are in flight in registers: while chunk c is multiplied from one LDS
  // buffer, chunk c+1 is written to the other and chunk c+1+kRing is loaded
  // into the register slot it leaves.  Each chunk is a short step, so a deep
  // ring is what keeps the memory round trips overlapped.
  const int which = tid / 256;  // 0: experts, 1: tokens
  const int sr = (tid % 256) / 4, sc = (tid % 4) * 16;
  const int64_t src = which == 0 ? int64_t(min(e0 + sr, E - 1)) * D : int64_t(min(t0 + sr, T - 1)) * D;
  const uint16_t *sbase = which == 0 ? wt : x;
  const bool ok = which == 0 ? e0 + sr < E : t0 + sr < T;
  const int C = D / kChunk / gridDim.z;  // chunks of this block's run
  const int c_base = bz * C;
  lt += int64_t(bz) * T * E;
  struct Stage { uint4 v0, v1; };
  auto load = [&](int c, Stage &st) __attribute__((always_inline)) {
    const uint4 *p = reinterpret_cast<const uint4 *>(sbase + src + (c_base + min(c, C - 1)) * kChunk + sc);
    st.v0 = p[0];
    st.v1 = p[1];
  };
  auto store = [&](int buf, const Stage &st) __attribute__((always_inline)) {
    // per-component select: a select of whole uint4 values goes through scratch
    auto keep = [&](uint4 v) { return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u); };
    *reinterpret_cast<uint4 *>(&sab[buf][which][sr][sc]) = keep(st.v0);
    *reinterpret_cast<uint4 *>(&sab[buf][which][sr][sc + 8]) = keep(st.v1);
  };
  constexpr int kRing = 2;  // even: LDS buffer of chunk c is c % 2
  Stage ring[kRing];  // slot c % kRing holds chunk c until it is written to LDS
#pragma unroll
  for (int u = 0; u < kRing; ++u) load(u, ring[u]);
  store(0, ring[0]);
  load(kRing, ring[0]);
  __syncthreads();
  // chunk c from LDS buffer buf; then chunk c+1 (held in nx) to the other
  // buffer, whose last readers (chunk c-1) are past the previous barrier, and
  // chunk c+1+kRing into nx.
  auto step = [&](int c, int buf, Stage &nx) __attribute__((always_inline)) {
    if constexpr (DT == kDtBF16) {
      bf16x8 av[2][2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          av[i][j] = *reinterpret_cast<const bf16x8 *>(&sab[buf][0][we * 32 + i * 16 + lr][lg * 16 + j * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *reinterpret_cast<const bf16x8 *>(&sab[buf][1][wtk * 16 + lr][lg * 16 + j * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i][0], bv[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i][1], bv[1], d, 0, 0, 0);
        acc[i] += d;
      }
    } else {
      // fp16: head/tail split of both operands, four products per pair
      bf16x8 ah[2][2], at[2][2], bh[2], bt[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          f16x8_split(*reinterpret_cast<const uint4 *>(&sab[buf][0][we * 32 + i * 16 + lr][lg * 16 + j * 8]),
                      ah[i][j], at[i][j]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        f16x8_split(*reinterpret_cast<const uint4 *>(&sab[buf][1][wtk * 16 + lr][lg * 16 + j * 8]), bh[j], bt[j]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i][j], bh[j], d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i][j], bt[j], d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at[i][j], bh[j], d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at[i][j], bt[j], d, 0, 0, 0);
        }
        acc[i] += d;
      }
    }
    store(buf ^ 1, nx);
    load(c + 1 + kRing, nx);
    __syncthreads();
  };
  for (int c = 0; c < C; c += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u)
      if (c + u < C) step(c + u, u & 1, ring[(u + 1) % kRing]);
  }
  const int t = t0 + wtk * 16 + lr;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int eb = e0 + we * 32 + i * 16 + lg * 4;
    const f32x4 v = acc[i];
    if (t < T) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (eb + q < E) lt[int64_t(t) * E + eb + q] = v[q] + (bias && bz == 0 ? bias[eb + q] : 0.0f);
    }
  }
}

// ---- 3. candidates, exact recomputation, selection -------------------------
struct CertArgs {
  const uint16_t *x, *wt;
  const float *bias, *lt, *wnorm;
  int T, D, E, K;
  int n_lt;  // partial L~ arrays, [n_lt][T][E] (1 or 2)
  float gamma;
  int32_t *idx_out;
  float *w_out;
  uint16_t *x16;  // nullable: fp16 staging copy of x for the 4-bit GEMMs
  int8_t *xsh;
  XgOut xo;       // and its group means (xo.xg nullable)
  int32_t *counts;  // nullable: dispatch counts [N / seg][E + 1] of the slots' experts, per segment of seg slots
  int seg;
};

// One wave per token; each lane keeps L~ of experts lane + 64*m, m < MPL.
template <int MPL, int DT>
__global__ __launch_bounds__(kThreads) void router_certify_kernel(CertArgs a) {
  constexpr int kNW = kThreads / kWave;
  constexpr int kBatch = 32;  // candidates recomputed per batch
  __shared__ float s_l[kNW][MPL * kWave];          // recomputed logits by list position
  __shared__ int32_t s_e[kNW][MPL * kWave];        // expert id by list position
  __shared__ float s_part[kNW][kBatch][kWave + 1];  // chunk partials of a batch (C <= 64)
  const int wv = threadIdx.x / kWave, lane = lane_id();
  const int t = blockIdx.x * kNW + wv;
  if (t >= a.T) return;  // whole waves
  const int E = a.E, D = a.D, K = a.K, C = D / kChunk;

  // L~ row, ||x_t||, max_e ||W_e||, max |bias|
  float lv[MPL];
#pragma unroll
  for (int m = 0; m < MPL; ++m) {
    const int e = lane + kWave * m;
    // both partials loaded unconditionally (the second from the first array
    // when there is one) so that all loads of the row are in flight together
    const int ec = min(e, E - 1);
    const float l0 = a.lt[int64_t(t) * E + ec];
    const float l1 = a.lt[(int64_t(a.n_lt > 1 ? a.T : 0) + t) * E + ec];
    lv[m] = e < E ? (a.n_lt > 1 ? l0 + l1 : l0) : -INFINITY;
  }
  // max_e ||W_e|| and max |bias| (loads in flight with those of x)
  float wn = 0.f, bmax = 0.f;
#pragma unroll
  for (int m = 0; m < MPL; ++m) {
    const int e = min(lane + kWave * m, E - 1);  // repeats of expert E-1 do not change a max
    wn = fmaxf(wn, a.wnorm[e]);
    if (a.bias) bmax = fmaxf(bmax, fabsf(a.bias[e]));
  }
  // ||x_t||^2: d <= 64 * 64 gives at most 8 pieces of 8 per lane, all loaded
  // together; the same registers give the fp16 staging row when asked.
  float xs = 0.f;
  RowF16 xr;
  row_f16_load(a.x + int64_t(t) * D, D, xr);
  {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if ((q * kWave + lane) * 8 < D) {
        const uint4 v = xr.v[q];
        const float f[8] = {half_lo<DT>(v.x), half_hi<DT>(v.x), half_lo<DT>(v.y), half_hi<DT>(v.y),
                            half_lo<DT>(v.z), half_hi<DT>(v.z), half_lo<DT>(v.w), half_hi<DT>(v.w)};
#pragma unroll
        for (int i = 0; i < 8; ++i) xs = __builtin_fmaf(f[i], f[i], xs);
      }
    }
  }
  xs = wave_sum(xs);
  if (a.x16) row_f16_store(xr, D, a.x16 + int64_t(t) * D, a.xsh + t, DT == kDtF16, a.xo, t);  // xr dies here
  wn = wave_max(wn);
  bmax = wave_max(bmax);
  const float bound = a.gamma * (sqrtf(xs) * sqrtf(wn) * 1.001f + bmax);

  // k-th largest L~ value
  float vk = 0.f;
  {
    uint32_t taken = 0;
    for (int j = 0; j < K; ++j) {
      const int be = wave_argmax<MPL>(lv, E, taken, vk);
      if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    }
  }
  const float thr = vk - 2.0f * bound;

  // candidate list (all experts when too many)
  int n = 0;
#pragma unroll
  for (int m = 0; m < MPL; ++m) {
    const int e = lane + kWave * m;
    n += __popcll(__ballot(e < E && lv[m] >= thr));
  }
  const bool all = n > kMaxCand;
  int pos[MPL];
  {
    int base = 0;
    const uint64_t lt_mask = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
    for (int m = 0; m < MPL; ++m) {
      const int e = lane + kWave * m;
      const bool c = e < E && (all || lv[m] >= thr);
      const uint64_t b = __ballot(c);
      pos[m] = c ? base + __popcll(b & lt_mask) : -1;
      if (c) s_e[wv][pos[m]] = e;
      base += __popcll(b);
    }
    n = base;
  }
  __builtin_amdgcn_wave_barrier();

  // Exact logits of the listed experts, kBatch at a time.  Lane (slot, ch)
  // runs the 64-long fma chain of chunk ch for candidates slot, slot+slots,
  // ... (two chains at a time); then lane p adds candidate p's C chunk
  // partials in chunk order.
  const int slots = kWave / C;
  const int slot = lane / C, ch = lane % C;
  const bool lane_on = slot < slots;
  float xf[kChunk];  // this lane's x chunk as fp32, widened once for all its chains
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 v = *reinterpret_cast<const uint4 *>(a.x + int64_t(t) * D + ch * kChunk + q * 8);
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      xf[8 * q + 2 * h] = half_lo<DT>(vw[h]);
      xf[8 * q + 2 * h + 1] = half_hi<DT>(vw[h]);
    }
  }
  // Lane (slot, ch) takes candidates slot, slot + slots, ...; the router row
  // chunk of the next one is loaded while the current chain runs.
  auto load_row = [&](int e, uint4 (&v)[8]) {
    const uint4 *wr = reinterpret_cast<const uint4 *>(a.wt + int64_t(e) * D + ch * kChunk);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = wr[q];
  };
  auto chain = [&](const uint4 (&v)[8]) -> float {
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t wv4[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        part = __builtin_fmaf(xf[8 * q + 2 * h], half_lo<DT>(wv4[h]), part);
        part = __builtin_fmaf(xf[8 * q + 2 * h + 1], half_hi<DT>(wv4[h]), part);
      }
    }
    return part;
  };
  for (int b0 = 0; b0 < n; b0 += kBatch) {
    const int nb = min(kBatch, n - b0);
    uint4 va[8], vb[8];
    int r = slot;
    load_row(s_e[wv][b0 + min(r, nb - 1)], va);
    // two candidates per turn, alternating buffers (no dynamic register indexing)
    for (; r < nb; r += 2 * slots) {
      load_row(s_e[wv][b0 + min(r + slots, nb - 1)], vb);
      const float pa = chain(va);
      if (lane_on) s_part[wv][r][ch] = pa;
      if (r + slots >= nb) break;
      load_row(s_e[wv][b0 + min(r + 2 * slots, nb - 1)], va);
      const float pb = chain(vb);
      if (lane_on) s_part[wv][r + slots][ch] = pb;
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < nb) {
      float acc = 0.f;
      for (int c = 0; c < C; ++c) acc = acc + s_part[wv][lane][c];
      const int e = s_e[wv][b0 + lane];
      s_l[wv][b0 + lane] = a.bias ? acc + a.bias[e] : acc;
    }
    __builtin_amdgcn_wave_barrier();
  }

  // top-k over the list.  List positions follow expert order, so the lower
  // position breaks ties exactly as the lower expert id.  A list of at most
  // 64 (the usual case) is ranked in one pass: lane p counts the entries that
  // come before its own (larger, or equal at a lower position).
  int my_p = 0;
  float my_l = 0.f, top = 0.f;
  if (n <= kWave) {
    __shared__ int32_t s_rank[kNW][kMaxTopK];  // list position of the rank-j entry
    const float mine = lane < n ? s_l[wv][lane] : -INFINITY;
    int rank = 0;
    for (int q = 0; q < n; ++q) {
      const float o = s_l[wv][q];
      rank += (o > mine || (o == mine && q < lane)) ? 1 : 0;
    }
    if (lane < n && rank < K) s_rank[wv][rank] = lane;
    __builtin_amdgcn_wave_barrier();
    top = s_l[wv][s_rank[wv][0]];
    if (lane < K) {
      my_p = s_rank[wv][lane];
      my_l = s_l[wv][my_p];
    }
  } else {
    float ll[MPL];  // list entry lane + 64*q
#pragma unroll
    for (int q = 0; q < MPL; ++q) {
      const int p = lane + kWave * q;
      ll[q] = p < n ? s_l[wv][p] : -INFINITY;
    }
    uint32_t taken = 0;
    for (int j = 0; j < K; ++j) {
      float bv;
      const int bp = wave_argmax<MPL>(ll, n, taken, bv);
      if ((bp & (kWave - 1)) == lane) taken |= 1u << (bp / kWave);
      if (j == 0) top = bv;
      if (lane == j) { my_p = bp; my_l = bv; }
    }
  }
  const int my_e = s_e[wv][my_p];

  // softmax: recomputed logits where listed, L~ elsewhere (cancels when renormalised)
  float z = 0.f;
#pragma unroll
  for (int m = 0; m < MPL; ++m) {
    const int e = lane + kWave * m;
    if (e < E) z += expf((pos[m] >= 0 ? s_l[wv][pos[m]] : lv[m]) - top);
  }
  z = wave_sum(z);
  const float pj = expf(my_l - top) / z;
  float psum = 0.f;
  for (int j = 0; j < K; ++j) psum = psum + read_lane(pj, j);
  if (lane < K) {
    a.idx_out[int64_t(t) * K + lane] = my_e;
    a.w_out[int64_t(t) * K + lane] = pj / psum;
    // integer sums: the same counts whatever the order of the additions
    if (a.counts) atomicAdd(&a.counts[((int64_t(t) * K + lane) / a.seg) * (E + 1) + my_e], 1);
  }
}

}  // namespace

bool route_mfma_applies(const moe_layer_desc *d, int32_t T) {
  // Below 64K (token, expert) logits the per-chunk vector router is faster:
  // the matrix-core router's three launches cost more than its fma chains.
  return d->act_dtype != MOE_DT_F32 && d->renormalize && d->d_model % kChunk == 0 &&
         d->d_model <= kWave * kChunk && T >= 64 && int64_t(T) * d->n_experts >= 65536;
}

bool route_counts_dispatch(const moe_layer_desc *d, int32_t T) {
  return route_mfma_applies(d, T) && dispatch_segment_slots(d, T) > 0;
}

// Prepared router: WT [E][D] (16-bit), then, from router_packed_norms_offset,
// the squared-norm partials [D/256][E] and their sums [E] (fp32), as the
// transpose kernel and the logit kernel leave them in the scratch.
bool router_pack_applies(const moe_layer_desc *d) {
  return d->act_dtype != MOE_DT_F32 && d->d_model % kChunk == 0 && d->d_model <= kWave * kChunk;
}
size_t router_packed_norms_offset(const moe_layer_desc *d) {
  return (size_t(d->n_experts) * d->d_model * 2 + 255) / 256 * 256;
}
size_t router_packed_bytes(const moe_layer_desc *d) {
  const size_t nkb = (d->d_model + 255) / 256;
  return router_packed_norms_offset(d) + (nkb + 1) * size_t(d->n_experts) * 4;
}

namespace {
// The sums of the squared-norm partials, in partial order (the order the
// logit kernel uses).
__global__ __launch_bounds__(kThreads) void router_norm_sum_kernel(float *normp, int n_kb, int E) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= E) return;
  float s = 0.f;
  for (int kb = 0; kb < n_kb; ++kb) s += normp[int64_t(kb) * E + e];
  normp[int64_t(n_kb) * E + e] = s;
}
}  // namespace

void launch_pack_router(const moe_layer_desc *d, const void *w_router, void *out, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = d->d_model, E = d->n_experts, nkb = (D + 255) / 256;
  uint16_t *wt = static_cast<uint16_t *>(out);
  float *normp = reinterpret_cast<float *>(static_cast<char *>(out) + router_packed_norms_offset(d));
  if (d->act_dtype == MOE_DT_F16)
    launch(router_transpose_kernel<kDtF16>, dim3((E + 63) / 64, nkb), dim3(kThreads), 0, s,
           static_cast<const uint16_t *>(w_router), D, E, wt, normp, static_cast<int32_t *>(nullptr), 0);
  else
    launch(router_transpose_kernel<kDtBF16>, dim3((E + 63) / 64, nkb), dim3(kThreads), 0, s,
           static_cast<const uint16_t *>(w_router), D, E, wt, normp, static_cast<int32_t *>(nullptr), 0);
  launch(router_norm_sum_kernel, dim3((E + kThreads - 1) / kThreads), dim3(kThreads), 0, s, normp, nkb, E);
}

// Scratch: L~ [T][E] f32, then WT [E][D] (16-bit), then norm partials [D/256][E]
// f32, each part starting on a 16-byte boundary (offsets in floats).
static int64_t align4(int64_t v) { return (v + 3) & ~int64_t(3); }

// Chunk runs of the matrix-core logits: two when the chunk count is even
// (more workgroups in flight; partial sums added by the certification).
static int route_mfma_splits(const moe_layer_desc *d) { return (d->d_model / kChunk) % 2 == 0 ? 2 : 1; }

int64_t route_mfma_scratch_floats(const moe_layer_desc *d, int32_t T) {
  const int64_t E = d->n_experts, D = d->d_model, nkb = (D + 255) / 256;
  return align4(route_mfma_splits(d) * int64_t(T) * E) + align4((E * D + 1) / 2) + (nkb + 1) * E;
}

namespace {
template <int DT>
void launch_route_mfma_t(const moe_layer_desc *d, int32_t T, const void *x, const void *w_router, const float *bias,
                         int32_t *idx, float *w, float *scratch, void *x16, int8_t *xsh, XgOut xo, hipStream_t s,
                         StageMarker *mk, int32_t *counts, int seg, const void *packed) {
  const int D = d->d_model, E = d->n_experts, nkb = (D + 255) / 256, C = D / kChunk;
  const int64_t N = int64_t(T) * d->top_k;
  const int n_counts = counts ? int((N + seg - 1) / seg * (E + 1)) : 0;
  float *lt = scratch;
  const int nz = route_mfma_splits(d);
  const int64_t o_wt = align4(nz * int64_t(T) * E), o_np = o_wt + align4((int64_t(E) * D + 1) / 2);
  const uint16_t *wt = reinterpret_cast<uint16_t *>(scratch + o_wt);
  float *normp = scratch + o_np;
  if (packed) {
    // the prepared router (moe_pack_router): the transposed weight and its
    // summed norms, read in place; no transpose kernel
    wt = static_cast<const uint16_t *>(packed);
    normp = reinterpret_cast<float *>(const_cast<char *>(static_cast<const char *>(packed)) +
                                      router_packed_norms_offset(d));
    launch(router_mfma_kernel<DT>, dim3((E + 63) / 64, (T + 63) / 64, nz), dim3(kMfThreads), 0, s,
           static_cast<const uint16_t *>(x), wt, bias, normp, nkb, T, D, E, lt, 1, counts, n_counts);
  } else {
    launch(router_transpose_kernel<DT>, dim3((E + 63) / 64, nkb), dim3(kThreads), 0, s,
           static_cast<const uint16_t *>(w_router), D, E, const_cast<uint16_t *>(wt), normp, counts, n_counts);
    launch(router_mfma_kernel<DT>, dim3((E + 63) / 64, (T + 63) / 64, nz), dim3(kMfThreads), 0, s,
           static_cast<const uint16_t *>(x), wt, bias, normp, nkb, T, D, E, lt, 0, nullptr, 0);
  }
  if (mk) mk->mark("route_mfma");
  // |L~ - L| <= gamma * S: the MFMAs of a chunk counted as 32 sequential
  // roundings each (two per chunk for bf16, eight for the fp16 head/tail
  // products), C chunk additions, and the fixed order's 64 + C + 1
  // roundings, with a margin: (256 + 2C) units of 2^-24 for bf16, (384 + 2C)
  // for fp16.
  const float gamma = float((DT == kDtF16 ? 384 : 256) + 2 * C) * 5.9604645e-8f;
  CertArgs ca{static_cast<const uint16_t *>(x), wt, bias, lt, normp + int64_t(nkb) * E, T, D, E, d->top_k, nz,
              gamma, idx, w, static_cast<uint16_t *>(x16), xsh, xo, counts, seg};
  const dim3 grid((T + kThreads / kWave - 1) / (kThreads / kWave)), block(kThreads);
  if (E <= 64) launch((router_certify_kernel<1, DT>), grid, block, 0, s, ca);
  else if (E <= 128) launch((router_certify_kernel<2, DT>), grid, block, 0, s, ca);
  else if (E <= 256) launch((router_certify_kernel<4, DT>), grid, block, 0, s, ca);
  else if (E <= 512) launch((router_certify_kernel<8, DT>), grid, block, 0, s, ca);
  else launch((router_certify_kernel<16, DT>), grid, block, 0, s, ca);
  if (mk) mk->mark("route_certify");
}

}  // namespace

void launch_route_mfma(const moe_layer_desc *d, int32_t T, const void *x, const void *w_router, const float *bias,
                       int32_t *idx, float *w, float *scratch, void *x16, int8_t *xsh, XgOut xo, void *stream,
                       StageMarker *mk, int32_t *counts, int seg, const void *packed) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (counts && seg <= 0) counts = nullptr;
  if (d->act_dtype == MOE_DT_F16)
    launch_route_mfma_t<kDtF16>(d, T, x, w_router, bias, idx, w, scratch, x16, xsh, xo, s, mk, counts, seg, packed);
  else
    launch_route_mfma_t<kDtBF16>(d, T, x, w_router, bias, idx, w, scratch, x16, xsh, xo, s, mk, counts, seg,
                                 packed);
}

}  // namespace moe
