// Standalone RoPE of bf16 latent rows ("Compressed Sparse Attention . ratio
// m = 4", Normalize + RoPE + cache; Released Flash configuration, RoPE
// sub-dimension 64): the last rope_dim features of each row turn as pairs
// (2i, 2i+1) by (cos, sin) column i of the row's table row, each exact value
// rounded once to bf16 (rope_pair). One thread per rotary pair; features
// outside the slice are copied when the output is another buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
  const int64_t half = a.rope_dim / 2;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = id / half;
  if (row >= a.rows) return;
  const int64_t i = id - row * half;
  const int64_t f = a.width - a.rope_dim + 2 * i;
  const uint16_t *src = a.in + row * a.width;
  const uint32_t pair = *reinterpret_cast<const uint32_t *>(src + f);
  const float2 cs = *reinterpret_cast<const float2 *>(a.rope_cs + (a.first_row + row) * a.rope_dim + 2 * i);
  uint32_t r0, r1;
  rope_pair(bf16_val(pair & 0xffffu), bf16_val(pair >> 16), cs.x, cs.y, r0, r1);
  uint16_t *dst = a.out + row * a.width;
  *reinterpret_cast<uint32_t *>(dst + f) = r0 | (r1 << 16);
  if (a.out != a.in) {
    // this thread's share of the unrotated features
    const int64_t rest = a.width - a.rope_dim;
    for (int64_t k = i; k < rest; k += half) dst[k] = src[k];
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, hipStream_t stream) {
  const int64_t total = a.rows * (a.rope_dim / 2);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_kernel, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvc
