// Residual correction of mlp_merge plans.
//
// "Technische Samenvatting: SparseSAM", Methodologie, 2. Residual-Consistency MLP,
// residual-propagation bullet: the tokens outside the keep-set bypass the MLP and pass
// the residual connection as y_i = x_i + eps_i. Reading taken for merging (the SparseSAM
// README's registry API names an mlp_merge flag): the keep-set's MLP updates are merged
// into one, their mean, and every real token of the segment outside the keep-set adds it.
//
// merge_kernel: one 256-thread workgroup per (segment, block of 64 channels). The
// segment's keep-set slots are marked in an LDS bit set; four thread groups sum the
// keep-set's updates of their channel over rows g, g + 4, ... in order, the four partial
// sums are added as (p0 + p1) + (p2 + p3) and divided by K; then the groups walk the
// segment's slots g, g + 4, ... and add the mean to every real unmarked slot's row.
// Every sum has a fixed order: the result is reproducible run to run.
#include "internal.hpp"

namespace sparsesam {

__global__ void __launch_bounds__(256) merge_kernel(float* __restrict__ x, const int* __restrict__ routed,
                                                    const float* __restrict__ upd, SegmentMap map, int C,
                                                    const int* __restrict__ seg_k, const int* __restrict__ seg_off,
                                                    int routed_per_image) {
  extern __shared__ uint32_t keep_bits[];  // one bit per slot of the segment
  __shared__ float part[4][64];
  const int seg = blockIdx.x, tid = threadIdx.x, g = tid >> 6, l = tid & 63;
  const int c = blockIdx.y * 64 + l;
  const int n = map.n;
  const int tokens = map.grid_h * map.grid_w;
  const int img = map.f_spi.div(seg), w = seg - img * map.segs_per_img;
  const int K = seg_k[w];
  const size_t base = (size_t)img * routed_per_image + seg_off[w];
  const int words = (n + 31) >> 5;
  for (int i = tid; i < words; i += 256) keep_bits[i] = 0u;
  __syncthreads();
  // slot of a keep-set row: its token inside the grid, or inside this segment's window
  const int wy = map.window ? w / map.nwx : 0, wx = map.window ? w - (w / map.nwx) * map.nwx : 0;
  for (int i = tid; i < K; i += 256) {
    const int tok = routed[base + i] - img * tokens;
    int slot = tok;
    if (map.window) {
      const int y = tok / map.grid_w, xx = tok - (tok / map.grid_w) * map.grid_w;
      slot = (y - wy * map.window) * map.window + (xx - wx * map.window);
    }
    if (slot >= 0 && slot < n) atomicOr(&keep_bits[slot >> 5], 1u << (slot & 31));
  }
  float s = 0.0f;
  if (c < C)
    for (int k = g; k < K; k += 4) s = s + upd[(base + k) * (size_t)C + c];
  part[g][l] = s;
  __syncthreads();
  const float mean = ((part[0][l] + part[1][l]) + (part[2][l] + part[3][l])) / (float)K;
  if (c >= C) return;
  for (int slot = g; slot < n; slot += 4) {
    if ((keep_bits[slot >> 5] >> (slot & 31)) & 1u) continue;
    const int row = map.row_of(seg, slot);
    if (row < 0) continue;
    float* px = x + (size_t)row * C + c;
    *px = *px + mean;
  }
}

hipError_t launch_merge(const sparsesam_plan& p, float* x, int batch, const int* routed, const float* upd,
                        hipStream_t st) {
  const int segs = batch * p.segs_per_img;
  if (segs <= 0) return hipSuccess;
  const size_t lds = (size_t)((p.n + 31) / 32) * 4;
  dim3 grid((unsigned)segs, (unsigned)((p.desc.channels + 63) / 64));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), lds, st, x, routed, upd, p.segmap(), p.desc.channels, p.d_seg_k,
                     p.d_seg_off, p.routed_per_image);
  return hipGetLastError();
}

}  // namespace sparsesam
