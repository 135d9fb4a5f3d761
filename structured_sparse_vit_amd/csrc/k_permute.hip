// Stripe-sort permutation and keep-set of every segment of an image.
//
// "Technische Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort Attention,
// stripe-sort bullet: tokens are sorted by importance, the sorted list is viewed as
// a matrix and transposed before flattening, which spreads the important tokens over
// the whole sequence. Part 2 (Residual-Consistency MLP), token routing bullet: the
// keep-set follows the same deterministic order.
//
// The order is total: importance descending (-0.0 == +0.0, NaN after every number,
// pad slots after every real slot), then slot ascending. A slot's rank is therefore
// the number of slots that precede it, and its stripe-sorted position follows from
// the rank alone: rank rho sits at stripe rho % g, offset rho / g, i.e. position
// (rho % g) * S + rho / g. No sorted list is ever materialised.
//
//  * rank_kernel: one workgroup per (segment, 64-slot chunk). Each wavefront counts,
//    for the chunk's 64 slots (one per lane), the preceding slots inside its share of
//    the segment's keys (held in LDS as 32-bit order keys); the shares are summed in
//    LDS and the 64 lanes of wavefront 0 write perm and inv. All 1024 threads of a
//    workgroup keep the GPU busy even for a single image (4096 slots -> 64 workgroups).
//  * keepset_kernel: one workgroup per image reads each real token's rank back from
//    inv, flags the K first of its segment, and compacts the flags in raster order
//    (block-wide scan), which gives the keep-set ascending.
#include <algorithm>

#include "internal.hpp"

namespace sparsesam {

// 32-bit key that orders descending importance ascending: larger value -> smaller key.
__device__ __forceinline__ uint32_t desc_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0xFFFFFFFEu;       // NaN: after every number
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;  // -0.0 -> +0.0
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}
constexpr uint32_t kPadKey = 0xFFFFFFFFu;  // pad slots: after every real slot

constexpr int kRankWaves = 16;

__global__ void __launch_bounds__(64 * kRankWaves) rank_kernel(const float* __restrict__ imp, SegmentMap map,
                                                               int n, int stripes, int chunks,
                                                               int* __restrict__ perm, int* __restrict__ inv) {
  extern __shared__ uint32_t key_lds[];  // keys of the segment, padded to a multiple of 16
  __shared__ int part[kRankWaves][64];
  const int seg = blockIdx.x / chunks, chunk = blockIdx.x - (blockIdx.x / chunks) * chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tokens = map.grid_h * map.grid_w;
  const int img = seg / map.segs_per_img;
  const float* im = imp + (size_t)img * tokens;
  const int n16 = (n + 15) & ~15;
  // keys past n are pad keys with index >= n: they never precede a real slot
#pragma unroll 4
  for (int s = tid; s < n16; s += blockDim.x) {
    const int row = s < n ? map.row_of(seg, s) : -1;
    key_lds[s] = row >= 0 ? desc_key(im[row - img * tokens]) : kPadKey;
  }
  __syncthreads();
  const int slot = chunk * 64 + lane;
  const bool valid = slot < n;
  const uint32_t mine = valid ? key_lds[slot] : 0u;
  // this wavefront's share of the keys, 16 at a time (four 16-byte broadcast reads in
  // flight per step)
  const int per = ((n16 / 16 + kRankWaves - 1) / kRankWaves) * 16;
  const int j0 = wave * per, j1 = min(n16, j0 + per);
  int cnt = 0;
  const uint4* k4 = reinterpret_cast<const uint4*>(key_lds);
  for (int j = j0; j < j1; j += 16) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = k4[j / 4 + u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t kk[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = j + 4 * u + e;
        cnt += (kk[e] < mine) | ((kk[e] == mine) & (jj < slot));
      }
    }
  }
  part[wave][lane] = cnt;
  __syncthreads();
  if (wave == 0 && valid) {
    int rank = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) rank += part[w][lane];
    const int S = n / stripes;
    const int p = (rank % stripes) * S + rank / stripes;
    const size_t base = (size_t)seg * n;
    perm[base + p] = slot;
    inv[base + slot] = p;
  }
}

__global__ void __launch_bounds__(1024) keepset_kernel(const int* __restrict__ inv, SegmentMap map, int segs, int n,
                                                       int stripes, const int* __restrict__ seg_k,
                                                       int routed_per_image, int* __restrict__ routed) {
  extern __shared__ unsigned char flag[];
  __shared__ int wave_tot[16];
  const int img = blockIdx.x;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int tokens = map.grid_h * map.grid_w;
  const int S = n / stripes;
  for (int t = tid; t < tokens; t += nth) flag[t] = 0;
  __syncthreads();
#pragma unroll 4
  for (int i = tid; i < segs * n; i += nth) {
    const int sg = i / n, s = i - sg * n;
    const int row = map.row_of(img * segs + sg, s) - img * tokens;
    if (row < 0 || row >= tokens) continue;  // pad slot
    const int p = inv[((size_t)img * segs + sg) * n + s];
    const int rank = stripes * (p % S) + p / S;
    if (rank < seg_k[sg]) flag[row] = 1;
  }
  __syncthreads();
  // compact the flags in raster order (block-wide exclusive scan)
  const int per = (tokens + nth - 1) / nth;
  const int t0 = tid * per;
  int cnt = 0;
  for (int t = t0; t < t0 + per && t < tokens; ++t) cnt += flag[t];
  const int lane = tid & 63, wv = tid >> 6;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wave_tot[w];
  int pos = before + incl - cnt;
  int* out = routed + (size_t)img * routed_per_image;
  for (int t = t0; t < t0 + per && t < tokens; ++t) {
    if (flag[t]) {
      if (pos < routed_per_image) out[pos] = img * tokens + t;
      ++pos;
    }
  }
}

size_t permute_lds_bytes(const sparsesam_plan& p) {
  const size_t tokens = (size_t)p.desc.grid_h * p.desc.grid_w;
  return std::max((size_t)((p.n + 15) & ~15) * 4, tokens);
}

hipError_t launch_permute(const sparsesam_plan& p, const float* imp, int batch, int* perm, int* inv, int* routed,
                          hipStream_t st) {
  const int chunks = (p.n + 63) / 64;
  const int segs = batch * p.segs_per_img;
  const size_t key_bytes = (size_t)((p.n + 15) & ~15) * 4;
  hipError_t e = hipFuncSetAttribute((const void*)rank_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)key_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rank_kernel, dim3((unsigned)(segs * chunks)), dim3(64 * kRankWaves), key_bytes, st, imp,
                     p.segmap(), p.n, p.desc.stripes, chunks, perm, inv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t flag_bytes = (size_t)p.desc.grid_h * p.desc.grid_w;
  e = hipFuncSetAttribute((const void*)keepset_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)flag_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(keepset_kernel, dim3(batch), dim3(1024), flag_bytes, st, inv, p.segmap(), p.segs_per_img, p.n,
                     p.desc.stripes, p.d_seg_k, p.routed_per_image, routed);
  return hipGetLastError();
}

}  // namespace sparsesam
