// pack.hip -- the tile-packed copy of an affine projection.
//
// The grouped matrix-core kernels multiply tiles of 16 weight rows and
// stream the reduction in slabs of 128 columns.  In the stored layout (row-
// major codes) a slab of a tile is 16 pieces of 64 or 128 bytes, one per row
// and a row apart; the packed layout stores each (tile, slab) as one
// contiguous block, so that a wave's loads of a slab read consecutive
// addresses:
//   codes[m][t][s][r][j] = w[m][16 t + r][SW s + j],  SW = 128 * b / 32 words,
// zero where SW s + j is past the row (a last slab of 64 columns).  Beside the
// codes it keeps each row's scales as exact fp16 values in the same (tile,
// slab) blocks, the group terms of the fast gate/up path in tile blocks, and
// one flag per matrix saying whether that path may run on it (the regions are
// described with PackedLayout).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kPackThreads = 256;

int64_t grid_for(int64_t n) { return std::max<int64_t>(1, std::min<int64_t>((n + kPackThreads - 1) / kPackThreads, 1 << 20)); }

// 16-byte pieces of the packed codes, grid-stride over all of them.
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const uint32_t *__restrict__ w,
                                                            uint32_t *__restrict__ out, int64_t pieces, int KW,
                                                            int nslab, int SW) {
  const int per_row = SW / 4;                       // pieces per (row, slab)
  const int64_t per_tile = int64_t(nslab) * 16 * per_row;
  for (int64_t q = int64_t(blockIdx.x) * kPackThreads + threadIdx.x; q < pieces;
       q += int64_t(gridDim.x) * kPackThreads) {
    const int64_t mt = q / per_tile;                // matrix * (N / 16) + tile
    int64_t rem = q - mt * per_tile;
    const int s = int(rem / (16 * per_row));
    rem -= int64_t(s) * 16 * per_row;
    const int r = int(rem / per_row), j = int(rem % per_row) * 4;
    const int64_t row = mt * 16 + r;                // row over all matrices (N % 16 == 0)
    const int col = s * SW + j;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (col < KW) v = *reinterpret_cast<const uint4 *>(w + row * KW + col);
    reinterpret_cast<uint4 *>(out)[q] = v;
  }
}

__global__ __launch_bounds__(kPackThreads) void pack_flags_init_kernel(int32_t *flags, int M) {
  const int m = blockIdx.x * kPackThreads + threadIdx.x;
  if (m < M) flags[m] = 1;
}

__device__ __forceinline__ float half16_to_f32(uint16_t v, bool f16) {
  return f16 ? f16_bits_to_f32(v) : bf16_bits_to_f32(v);
}

// Scales, [m][t][s][r][g'] from [m][group][n]: group = s*GPS + g', n = 16t + r.
// A scale that is neither 0 nor an fp16-exact value in [2^-14, 32] clears
// its matrix's flag (each such writer stores the same 0).
__global__ __launch_bounds__(kPackThreads) void pack_scales_kernel(const uint16_t *__restrict__ sc,
                                                                   uint16_t *__restrict__ out, int32_t *flags,
                                                                   int64_t n_out, int N, int G, int nslab, int GPS,
                                                                   int f16) {
  const int NT = N / 16;
  for (int64_t q = int64_t(blockIdx.x) * kPackThreads + threadIdx.x; q < n_out;
       q += int64_t(gridDim.x) * kPackThreads) {
    const int gq = int(q % GPS);
    int64_t rest = q / GPS;
    const int r = int(rest % 16);
    rest /= 16;
    const int s = int(rest % nslab);
    rest /= nslab;
    const int t = int(rest % NT);
    const int64_t m = rest / NT;
    const int group = s * GPS + gq, n = 16 * t + r;
    uint16_t o = 0;
    if (group < G) {
      const float v = half16_to_f32(sc[(m * G + group) * N + n], f16 != 0);
      const _Float16 h = static_cast<_Float16>(v);
      const float a = fabsf(v);
      const bool ok = static_cast<float>(h) == v && (v == 0.f || (a >= 0x1p-14f && a <= 32.f));
      if (!ok) flags[m] = 0;
      o = __builtin_bit_cast(uint16_t, h);
    }
    out[q] = o;
  }
}

// Group terms, [m][t][r][g] from the scales and biases [m][g][n]:
// round((b - 1024 s - n2) * group) with n2 = round(-(1024 + z) s), the part of
// each weight s q + b of the group that the kernels' expansion
// round(s (q - z) + delta) leaves out.  -(1024 + z) s is exact in fp32 (s has
// at most 11 significant bits, 1024 + z at most 8), so n2 is its one rounding
// to fp16, as the kernels' pk_mul gives it; b - 1024 s - n2 is exact in
// double.  A term that is not finite or reaches 2^15 clears the flag.
__global__ __launch_bounds__(kPackThreads) void pack_groups_kernel(const uint16_t *__restrict__ sc,
                                                                   const uint16_t *__restrict__ bi,
                                                                   uint16_t *__restrict__ out, int32_t *flags,
                                                                   int64_t n_out, int N, int G, int GP, int gs,
                                                                   float off, int f16) {
  const int NT = N / 16;
  for (int64_t q = int64_t(blockIdx.x) * kPackThreads + threadIdx.x; q < n_out;
       q += int64_t(gridDim.x) * kPackThreads) {
    const int g = int(q % GP);
    int64_t rest = q / GP;
    const int r = int(rest % 16);
    rest /= 16;
    const int t = int(rest % NT);
    const int64_t m = rest / NT;
    uint16_t o = 0;
    if (g < G) {
      const int64_t at = (m * G + g) * N + 16 * t + r;
      const float s = half16_to_f32(sc[at], f16 != 0), b = half16_to_f32(bi[at], f16 != 0);
      const float n2 = static_cast<float>(static_cast<_Float16>(off * s));
      const double c = (double(b) - 1024.0 * double(s) - double(n2)) * double(gs);
      if (!(fabs(c) < 32768.0)) flags[m] = 0;  // also NaN
      o = __builtin_bit_cast(uint16_t, static_cast<_Float16>(static_cast<float>(c)));
    }
    out[q] = o;
  }
}

}  // namespace

void launch_pack(const moe_layer_desc *d, int32_t proj, const uint32_t *w, const uint16_t *scales,
                 const uint16_t *biases, void *w_packed, void *stream) {
  PackedLayout L;
  if (!packed_layout(d, proj, &L)) return;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int b = d->w_format == MOE_WF_AFFINE_Q8 ? 8 : 4;
  const int KW = L.K * b / 32;
  const int M = d->n_experts + d->n_shared;
  const int f16 = d->act_dtype == MOE_DT_F16;
  unsigned char *base = static_cast<unsigned char *>(w_packed);
  uint32_t *codes = reinterpret_cast<uint32_t *>(base + L.codes);
  uint16_t *sc = reinterpret_cast<uint16_t *>(base + L.scales);
  uint16_t *bi = reinterpret_cast<uint16_t *>(base + L.biases);
  int32_t *flags = reinterpret_cast<int32_t *>(base + L.flags);
  const int64_t pieces = int64_t(M) * L.N * L.nslab * L.SW / 4;
  if (pieces <= 0) return;
  launch(pack_kernel, dim3(unsigned(grid_for(pieces))), dim3(kPackThreads), 0, st, w, codes, pieces, KW, L.nslab,
         L.SW);
  launch(pack_flags_init_kernel, dim3(unsigned((M + kPackThreads - 1) / kPackThreads)), dim3(kPackThreads), 0, st,
         flags, M);
  const int64_t n_sc = int64_t(M) * L.N * L.nslab * L.GPS;
  launch(pack_scales_kernel, dim3(unsigned(grid_for(n_sc))), dim3(kPackThreads), 0, st, scales, sc, flags, n_sc,
         L.N, L.G, L.nslab, L.GPS, f16);
  const int64_t n_bi = int64_t(M) * L.N * L.GP;
  const float off = b == 8 ? -1152.0f : -1032.0f;  // -(1024 + z)
  launch(pack_groups_kernel, dim3(unsigned(grid_for(n_bi))), dim3(kPackThreads), 0, st, scales, biases, bi, flags,
         n_bi, L.N, L.G, L.GP, d->group_size, off, f16);
}

}  // namespace moe
