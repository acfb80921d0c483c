// fp32 projection GEMM of the compressor on gfx950 matrix cores: the
// instances used by the library (kernel template in gemm_f32_kernel.h).
//
// Prefill picks by problem size:
//   256 x 256 tiles (eight 64 x 128 wavefronts, one workgroup per CU, 129 KiB
//     of LDS, double-buffered 32-deep k tiles) when there are at least 512
//     such tiles (two full rounds on 256 CUs);
//   otherwise 128 x 128 tiles (four 64 x 64 wavefronts, two workgroups per
//     CU) with a single 64-deep LDS k tile fed by a register prefetch, or
//     with the double-buffered 32-deep tiles when k is not a multiple of 64.
// At the long-prefill shape both large variants run at 86-87% of the fp32
// matrix peak.
// Tiles are remapped so each XCD walks a contiguous range of row tiles with
// the column tiles fastest (an A row tile is then reused from that XCD's L2).
// Decode (M = batch): decode_gemm_kernel, 32 columns per workgroup with the K
// range split over workgroups (each split writes its own partial sums) and
// over the wavefronts of a workgroup (summed in LDS).
#include "gemm_f32_kernel.h"

namespace kvc {

hipError_t launch_gemm(const GemmArgs &g, GemmShape shape, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  if (shape == GemmShape::kDecode) return gemm::launch_decode_gemm(g, stream);
  const int64_t m256 = (g.m + 255) / 256;
  if (g.n_half % 256 == 0 && m256 * (2 * g.n_half / 256) >= 512)
    return gemm::launch_tiled<256, 256, 64, 128, 8, false, 1>(g, stream);
  if (g.k % 64 == 0) return gemm::launch_sb<128, 128, 64, 64, 4, 64, 2>(g, stream);
  return gemm::launch_tiled<128, 128, 64, 64, 4, false, 2>(g, stream);
}

}  // namespace kvc
