// fp32 projection GEMM of the compressor on gfx950 matrix cores: the
// instances used by the library (kernel template in gemm_f32_kernel.h).
//
// Prefill picks by problem size (all direct-to-LDS, double-buffered 32-deep
// k stages):
//   256 x 256 tiles (eight 64 x 128 wavefronts, one workgroup per CU, 128 KiB
//     of LDS, last k-slice deferred past the barrier) when there are at least
//     512 such tiles (two full rounds on 256 CUs): 92% of the fp32 matrix
//     peak at the long-prefill shape;
//   256 x 128 tiles (eight 64 x 64 wavefronts) when there are at least 256;
//   128 x 128 tiles (four 64 x 64 wavefronts, two workgroups per CU) below.
// Tiles are remapped so each XCD walks a contiguous range of row tiles with
// the column tiles fastest (an A row tile is then reused from that XCD's L2).
// Every instance sums each output as p0 + p1 over the two k halves
// (gemm_f32_kernel.h), the order decode_f32.hip reproduces for one token.
// Decode from bf16 rows (M = batch): decode_gemm_kernel, 32 columns per
// workgroup with the K range split over workgroups (each split writes its
// own partial sums) and over the wavefronts of a workgroup (summed in LDS).
#include "gemm_f32_kernel.h"

namespace kvc {

hipError_t launch_gemm(const GemmArgs &g, GemmShape shape, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  if (shape == GemmShape::kDecode) return gemm::launch_decode_gemm(g, stream);
  const int64_t m256 = (g.m + 255) / 256;
  if (g.n_half % 256 == 0 && m256 * (2 * g.n_half / 256) >= 512)
    return gemm::launch_tiled<256, 256, 64, 128, 8, 1, true>(g, stream);
  if (g.n_half % 128 == 0 && m256 * (2 * g.n_half / 128) >= 256)
    return gemm::launch_tiled<256, 128, 64, 64, 8, 1, false>(g, stream);
  return gemm::launch_tiled<128, 128, 64, 64, 4, 2, false>(g, stream);
}

hipError_t launch_gemm_pool(const GemmArgs &g, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  return gemm::launch_pooling(g, stream);
}

}  // namespace kvc
