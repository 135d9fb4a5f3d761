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

// Strip kernel for patch 16: one 1024-thread workgroup per 16 tokens of one token row
// (a 16 x 256-pixel strip). The strip and its one-pixel halo (18 x 258 floats) are
// staged in LDS with coalesced loads. Each thread then computes four neighbouring pixel
// magnitudes from three 6-wide windows of the tile (16-byte LDS reads) into mag; 256
// threads sum the patch rows left to right, and 16 threads the row sums top to bottom
// -- the same operations in the same order as the per-token kernel above.
constexpr int kStripW = 256, kHaloW = kStripW + 2, kTileLd = 260;  // tile rows 16-byte aligned

__global__ void __launch_bounds__(1024) sobel_pool_strip_kernel(const float* __restrict__ img, int height, int width,
                                                                float* __restrict__ imp) {
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) float tile[18][kTileLd];
  __shared__ float mag[16][kStripW + 1];  // odd row stride: the row sums read 64 distinct banks
  __shared__ float rowsum[16][17];
  const int x0 = blockIdx.x * kStripW, ty = blockIdx.y, b = blockIdx.z;
  const int y0 = ty * 16;
  const float* P = img + (size_t)b * height * width;
  // every load of the strip is issued before the first LDS store (addresses clamped
  // into the image, values outside it replaced by zero afterwards)
  constexpr int kFill = 18 * kHaloW, kIters = (kFill + 1023) / 1024;
  float fv[kIters];
  bool inside[kIters];
#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    const int i = threadIdx.x + 1024 * k;
    const int rr = i / kHaloW, cc = i - (i / kHaloW) * kHaloW;
    const int yy = y0 - 1 + rr, xx = x0 - 1 + cc;
    const int cy = min(max(yy, 0), height - 1), cx = min(max(xx, 0), width - 1);
    fv[k] = P[(size_t)cy * width + cx];
    inside[k] = (yy >= 0) & (yy < height) & (xx >= 0) & (xx < width);
  }
#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    const int i = threadIdx.x + 1024 * k;
    if (i < kFill) tile[i / kHaloW][i - (i / kHaloW) * kHaloW] = inside[k] ? fv[k] : 0.0f;
  }
  __syncthreads();
  {
    // pixels (r, 4q + i), i < 4: tile rows r .. r + 2, tile columns 4q + i .. 4q + i + 2
    const int r = threadIdx.x >> 6, q = threadIdx.x & 63;
    float w[3][6];
#pragma unroll
    for (int dy = 0; dy < 3; ++dy) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&tile[r + dy][4 * q]);
      const float b0 = tile[r + dy][4 * q + 4], b1 = tile[r + dy][4 * q + 5];
      w[dy][0] = a[0];
      w[dy][1] = a[1];
      w[dy][2] = a[2];
      w[dy][3] = a[3];
      w[dy][4] = b0;
      w[dy][5] = b1;
    }
    const float two = 2.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gx = ((w[0][i + 2] + two * w[1][i + 2]) + w[2][i + 2]) - ((w[0][i] + two * w[1][i]) + w[2][i]);
      float gy = ((w[2][i] + two * w[2][i + 1]) + w[2][i + 2]) - ((w[0][i] + two * w[0][i + 1]) + w[0][i + 2]);
      float sq = gx * gx;
      float sq2 = gy * gy;
      sq = sq + sq2;
      mag[r][4 * q + i] = __builtin_sqrtf(sq);
    }
  }
  __syncthreads();
  if (threadIdx.x < 256) {
    const int tl = threadIdx.x >> 4, r = threadIdx.x & 15;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc = acc + mag[r][tl * 16 + c];
    rowsum[tl][r] = acc;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float tot = 0.0f;
    for (int i = 0; i < 16; ++i) tot = tot + rowsum[threadIdx.x][i];
    const int gw = width / 16;
    imp[(size_t)b * (height / 16) * gw + ty * gw + blockIdx.x * 16 + threadIdx.x] = tot / 256.0f;
  }
}

hipError_t launch_importance(const float* img, int batch, int height, int width, int patch, float* imp,
                             hipStream_t st) {
  if (patch == 16 && width % kStripW == 0) {
    dim3 grid(width / kStripW, height / 16, batch);
    hipLaunchKernelGGL(sobel_pool_strip_kernel, grid, dim3(1024), 0, st, img, height, width, imp);
    return hipGetLastError();
  }
  dim3 grid(width / patch, height / patch, batch);
  hipLaunchKernelGGL(sobel_pool_kernel, grid, dim3(patch * patch), 0, st, img, height, width, patch, imp);
  return hipGetLastError();
}

}  // namespace sparsesam
