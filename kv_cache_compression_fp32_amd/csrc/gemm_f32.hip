// fp32 projection GEMM of the compressor on gfx950 matrix cores: the
// instances used by the library (kernel template in gemm_f32_kernel.h).
//
// Prefill picks the largest tile that still fills the chip:
//   256 x 256 (eight 64 x 128 wavefronts, one workgroup per CU, 129 KiB of
//     LDS) when there are at least 512 such tiles (two full rounds on 256
//     CUs); about 86% of the fp32 matrix peak at the long-prefill shape;
//   256 x 128 (eight 64 x 64 wavefronts) when there are at least 256;
//   128 x 128 (four 64 x 64 wavefronts, two workgroups per CU) otherwise.
// Tiles are remapped so each XCD walks a contiguous range of row tiles with
// the column tiles fastest (an A row tile is then reused from that XCD's L2).
// Decode (M = batch): 64 x 64 tiles with the K range split so that about 512
// workgroups share the weights; each split writes its own partial sums.
#include "gemm_f32_kernel.h"

namespace kvc {

hipError_t launch_gemm(const GemmArgs &g, GemmShape shape, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  if (shape == GemmShape::kDecode) return gemm::launch_tiled<64, 64, 32, 32, 4, false, 2>(g, stream);
  const int64_t m256 = (g.m + 255) / 256;
  if (g.n_half % 256 == 0 && m256 * (2 * g.n_half / 256) >= 512) return gemm::launch_tiled<256, 256, 64, 128, 8, false, 1>(g, stream);
  if (m256 * (2 * g.n_half / 128) >= 256) return gemm::launch_tiled<256, 128, 64, 64, 8, false, 1>(g, stream);
  return gemm::launch_tiled<128, 128, 64, 64, 4, false, 2>(g, stream);
}

}  // namespace kvc
