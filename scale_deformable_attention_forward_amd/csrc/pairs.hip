// The head-pair layout of a bf16 value (MSDA_BF16_PAIRS): per image
// [nH][Nv][2][32], line (h, p) = pixel p of head h, then pixel p + 1.  The
// bilinear sample's two corners in one row of a level ("BEV(三) BEVFormer：
// Query 参数如何与 Feature 的 8 个 Head 交互", section 6) are then one
// 128-byte line, which the SCA gather fetches with one load per head.
//
// msda_pack_pairs_bf16's kernel: a copy from [n_images][Nv][nH][32].  Each
// thread writes one 16-byte chunk of the destination, so that a wave's
// stores cover 1 KiB of consecutive lines; chunk k of line (h, p) is octet
// k % 4 of pixel p + k / 4 (zeros past the image's last pixel).
#include "common.hpp"
#include "internal.hpp"

namespace msda {

__global__ __launch_bounds__(256) void pack_pairs_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t n_images, int64_t Nv, int nH) {
  const int64_t lines_per_image = Nv * nH;
  const int64_t chunks = n_images * lines_per_image * 8;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < chunks; e += step) {
    const int64_t line = e >> 3;
    const int k = (int)(e & 7);
    const int64_t img = line / lines_per_image;
    const int64_t rem = line - img * lines_per_image;
    const int64_t h = rem / Nv;
    const int64_t pix = rem - h * Nv + (k >> 2);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (pix < Nv) v = src[((img * Nv + pix) * nH + h) * 4 + (k & 3)];
    dst[e] = v;
  }
}

hipError_t launch_pack_pairs(const void* value, void* pairs, int64_t n_images, int64_t Nv, int nH,
                             hipStream_t stream) {
  const int64_t chunks = n_images * Nv * nH * 8;
  int64_t blocks = (chunks + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  pack_pairs_kernel<<<(unsigned)blocks, 256, 0, stream>>>(static_cast<const uint4*>(value), static_cast<uint4*>(pairs),
                                                          n_images, Nv, nH);
  return hipGetLastError();
}

}  // namespace msda
