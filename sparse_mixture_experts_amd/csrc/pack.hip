// pack.hip -- the tile-packed copy of an affine projection's codes.
//
// The grouped matrix-core kernels multiply tiles of 16 weight rows and
// stream the reduction in slabs of 128 columns.  In the stored layout
// (row-major codes) a slab of a tile is 16 pieces of 64 or 128 bytes, one per
// row and a row apart; the packed layout stores each (tile, slab) as one
// contiguous block, so that a wave's loads of a slab read consecutive
// addresses:
//   packed[m][t][s][r][j] = w[m][16 t + r][SW s + j],  SW = 128 * b / 32 words,
// zero where SW s + j is past the row (a last slab of 64 columns).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kPackThreads = 256;

// 16-byte pieces of the packed copy, grid-stride over all of them.
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

}  // namespace

void launch_pack(const moe_layer_desc *d, int32_t proj, const uint32_t *w, uint32_t *w_packed, void *stream) {
  int N = 0, K = 0;
  if (!proj_shape(d, proj, &N, &K)) return;
  const int b = d->w_format == MOE_WF_AFFINE_Q8 ? 8 : 4;
  const int KW = K * b / 32, SW = 128 * b / 32, nslab = (K + 127) / 128;
  const int64_t pieces = packed_words(d, proj) / 4;
  if (pieces <= 0) return;
  const int64_t blocks = std::min<int64_t>((pieces + kPackThreads - 1) / kPackThreads, 1 << 20);
  launch(pack_kernel, dim3(unsigned(blocks)), dim3(kPackThreads), 0, static_cast<hipStream_t>(stream), w, w_packed,
         pieces, KW, nslab, SW);
}

}  // namespace moe
