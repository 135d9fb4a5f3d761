// Token importance: Sobel gradient magnitude pooled per patch.
//
// "Technische Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort Attention
// (gradient-based ordering bullet): a parameter-free Sobel operator gives the local
// gradient magnitude, used as a proxy for information density. The result decides
// an integer permutation, so every operation is fp32 with one rounding in a fixed
// order (no contraction into fused multiply-adds, correctly rounded sqrt and divide).
//
// One workgroup per token: patch^2 threads each compute one pixel magnitude into
// LDS, then the patch rows are summed left to right and the row sums top to bottom.
// The kernel reads 4 bytes per pixel (plus halo hits in cache) and writes 4 bytes per
// token; it is latency-bound at these sizes (4 MiB per 1024 x 1024 image).
#include "internal.hpp"

namespace sparsesam {

__global__ void __launch_bounds__(1024) sobel_pool_kernel(const float* __restrict__ img, int height, int width,
                                                          int patch, float* __restrict__ imp) {
#pragma clang fp contract(off)
  __shared__ float mag[32 * 32];
  __shared__ float rowsum[32];
  const int gw = width / patch;
  const int tx = blockIdx.x, ty = blockIdx.y, b = blockIdx.z;
  const float* P = img + (size_t)b * height * width;
  const int r = threadIdx.x / patch, c = threadIdx.x - (threadIdx.x / patch) * patch;
  const int y = ty * patch + r, x = tx * patch + c;

  auto at = [&](int yy, int xx) -> float {
    return (yy >= 0 && yy < height && xx >= 0 && xx < width) ? P[(size_t)yy * width + xx] : 0.0f;
  };
  const float two = 2.0f;
  float gx = ((at(y - 1, x + 1) + two * at(y, x + 1)) + at(y + 1, x + 1)) -
             ((at(y - 1, x - 1) + two * at(y, x - 1)) + at(y + 1, x - 1));
  float gy = ((at(y + 1, x - 1) + two * at(y + 1, x)) + at(y + 1, x + 1)) -
             ((at(y - 1, x - 1) + two * at(y - 1, x)) + at(y - 1, x + 1));
  float sq = gx * gx;
  float sq2 = gy * gy;
  sq = sq + sq2;
  mag[r * patch + c] = __builtin_sqrtf(sq);
  __syncthreads();
  if (threadIdx.x < patch) {
    float acc = 0.0f;
    for (int i = 0; i < patch; ++i) acc = acc + mag[threadIdx.x * patch + i];
    rowsum[threadIdx.x] = acc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.0f;
    for (int i = 0; i < patch; ++i) tot = tot + rowsum[i];
    imp[(size_t)b * (height / patch) * gw + ty * gw + tx] = tot / (float)(patch * patch);
  }
}

hipError_t launch_importance(const float* img, int batch, int height, int width, int patch, float* imp,
                             hipStream_t st) {
  dim3 grid(width / patch, height / patch, batch);
  hipLaunchKernelGGL(sobel_pool_kernel, grid, dim3(patch * patch), 0, st, img, height, width, patch, imp);
  return hipGetLastError();
}

}  // namespace sparsesam
